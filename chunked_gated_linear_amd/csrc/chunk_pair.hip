// chunk_pair.hip -- bf16 chunked forward pass as two kernels: an intra-tile
// kernel, parallel over every pair of 16-token tiles, and an inter-tile kernel
// that carries the state across the sequence.
//
// Method: the sequence is cut into 16-token tiles; inside a tile the token
// interactions (K K^T, Q K^T) and the "historical state -> current token"
// products (K H, Q H) run on the matrix cores, and the state is carried from
// tile to tile ("Deep Dive: The Next Generation of Ultra-Long Context Sparse
// MoE LLMs", sec. 3.2; "Core Technologies Behind Ultra-Long-Context Sparse MoE
// Large Models", sec. 2.1).  The state h = S^T (d_k x d_v) is carried across
// pairs of tiles a, b (32 tokens).  With G the running sum of g over the pair,
// gamma = exp(G), delta_p = exp(G_31 - G_p), Gamma = exp(G_31):
//     A   = [[A00, 0], [A10, A11]],  A[t][s] = beta_t exp(G_t - G_s) k_t.k_s (s < t)
//     T   = (I + A)^-1 = [[T00, 0], [T10, T11]],  T10 = -T11 A10 T00
//     Tb  = T diag(beta),  P[t][s] = exp(G_t - G_s) q_t.k_s (s <= t)
//     U   = Tb (V - diag(gamma) K H)
//     O   = diag(gamma) Q H + P U
//     H'  = Gamma H + K^T diag(delta) U
// Everything but U, O and H' is independent of the state.  Only exponentials
// of non-positive numbers appear, so with the bounded gate every in-tile
// factor lies in [exp(-32 G), 1] and no reciprocal is formed.
//
// chunk_prep_kernel (intra-tile) -- one wave per (sequence, head, pair): gate,
//   in-pair cumulative sum, K K^T and K Q^T on MFMA, decay masks, the two
//   16 x 16 unit-triangular solves in fp32, T10 on fp32 MFMA, and hi/lo bf16
//   splits of Tb and P.  Its results (6.5 KB per pair) go to a workspace in
//   HBM, computed once per head rather than once per d_v slice.
// chunk_state_kernel (inter-tile) -- one workgroup per (sequence, head, one
//   or two slices of 16 columns of d_v), 2 SPW + 2 waves:
//   "chain" (one per slice)  the fp32 state slice (d_k x 16) in registers;
//                    per pair: K H, U, the 32-deep state update, all on MFMA;
//   "output" (one per slice) diag(gamma) Q H + P U on MFMA and the bf16
//                    stores, one pair behind the chain; q comes through the
//                    loader, P and gamma straight from global memory, several
//                    pairs ahead;
//   "loader"         streams k, q, v and the chain's part of the workspace
//                    into a ring of LDS records with direct global->LDS loads,
//                    a few pairs ahead of the chain;
//   "prefetch"       touches the lines of a pair further ahead so that the
//                    loader's requests hit L2: the workgroups of a head split
//                    the lines between them, one 4-byte load per line.
//   One workgroup barrier per pair.  The state (bf16) and U reach the output
//   wave through LDS, double buffered by pair parity.  Two slices share one
//   workgroup only when one slice per workgroup would need more than one
//   round of workgroups; then they share the loader's traffic.
//
// Precision: Tb, P and U are split into bf16 hi + lo parts and contracted as
// [X_hi | X_lo] . [Y ; Y] in one 32-deep MFMA (the issue cost of a 16-deep
// product).  The state is kept in fp32; its bf16 copy feeds K H and Q H.
//
// State row order.  Accumulator tile t = 2s + h of the state holds, in lane
// (n, grp) register i, row rho = 32 s + 8 grp + 4 h + i of the d_k x 16 slice;
// every 32-deep fragment of K or Q is then 8 consecutive elements of a row and
// two accumulator tiles form the 32-deep B fragment of H directly.
#include "la_device.h"
#include "la_launch.h"

namespace la {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Workspace record of one pair of tiles of one (sequence, head), in bytes.
// Fragment fields hold 64 lanes x 16 B in lane order.  With raw inputs (q and
// k to be normalised here) the per-token factors 1/|k_t| and 1/|q_t| are
// folded into the record: into A and P, into gamma and delta (the chain's K H
// and K^T updates use the raw k), and into the output's gamma (GMQ, the raw
// q); without them GMQ equals gamma.
struct WsRec {
  static constexpr int TB0 = 0;       // [Tb00 hi | Tb00 lo]   row n, columns 4grp..4grp+3
  static constexpr int TB1H = 1024;   // [Tb10 hi | Tb11 hi]
  static constexpr int TB1L = 2048;   // [Tb10 lo | Tb11 lo]
  static constexpr int PF0 = 3072;    // [P00 hi  | P00 lo]
  static constexpr int PF1H = 4096;   // [P10 hi  | P11 hi]
  static constexpr int PF1L = 5120;   // [P10 lo  | P11 lo]
  static constexpr int GM = 6144;     // gamma[32]  f32
  static constexpr int DL = 6272;     // delta[32]  f32
  static constexpr int GC = 6400;     // Gamma      f32
  static constexpr int GMQ = 6528;    // gamma[32] for the output, f32 (record padded to 256 B)
  static constexpr int BYTES = 6656;
};

// Rows of k or q in LDS: a 1 KB block holds 16 token rows x 64 B (32 elements
// of d_k); 16-byte chunk g of row t sits in slot rslot(t, g) = 4 t + (g ^ sw(t)),
// sw(t) = (t >> 1) & 3.  A direct-to-LDS load fills a block with lanes in slot
// order, so each 16-lane quarter of the load covers 4 whole 64-byte rows (a
// quarter spanning 16 rows costs the address unit about three times as much);
// the XOR keeps the fragment reads (row n, chunk grp in lane (n, grp)) free of
// bank conflicts.
__device__ inline int rsw(int t) { return (t >> 1) & 3; }
__device__ inline int rslot(int t, int g) { return 4 * t + (g ^ rsw(t)); }

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

// Wave-local ordering of LDS traffic (a wave's LDS operations execute in
// order; this keeps the compiler from reordering across the point).
__device__ inline void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s_waitcnt with only the vector-memory count limited (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ inline void wait_vmcnt() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }  // vmcnt 63, expcnt 7, lgkmcnt 0

// Workgroup barrier without the implicit "wait for every outstanding memory
// operation" of __syncthreads: callers wait for exactly what the other waves
// will read.  The wavefront fences only stop the compiler from moving memory
// accesses across the barrier.
__device__ inline void wg_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Direct global -> LDS loads: lane i's `bytes` land at lds + i * bytes.
__device__ inline void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// ============================================================== intra-tile

constexpr int kPrepWaves = 4;
constexpr int kPrepScr = 2560;   // per wave: A00 (then T00), A11 (then T11), beta[32], G[32],
                                 // 1/|k|[32], 1/|q|[32]
constexpr int kPrepRows = 8192;  // per wave: one pair's rows of k or q, as fragment blocks

constexpr int kPrepLDS = kPrepWaves * (kPrepScr + kPrepRows);

// Arguments of the intra-tile work over tokens [0, T) of each sequence; the
// pointers may be advanced to a later token, TB is the full sequence length
// (the stride between sequences, in tokens).
struct PrepArgs {
  const __bf16* q;
  const __bf16* k;
  const float* gate;
  const float* beta;
  char* ws;
  int gate_logit;
  float G;
  int B, T, TB, H;
  // Raw inputs: q and k are L2-normalised per token here (a zero vector stays
  // zero) and beta holds logits, beta = sigmoid(x).
  int raw;
  // Packed sequences (cu != nullptr): B sequences, sequence s holds tokens
  // [cu[s], cu[s+1]) of one packed sequence of TB tokens, and its pair p has
  // workspace record slot(s, p) = floor(cu[s] / 32) + s + p of nslot per head.
  const int* cu;
  int nslot;
  // Affine gate pre-activation (logit mode): the logit of head h is
  // gsc[h] * x + gbi[h] (NULL: scale 1, shift 0).
  const float* gsc;
  const float* gbi;
};

// Token range of packed sequence s, clamped to [0, TB] (so that out-of-order
// offsets stay memory-safe).
__device__ inline int seq_begin(const int* cu, int s, int TB) { return min(max(cu[s], 0), TB); }
__device__ inline int seq_end(const int* cu, int s, int TB) {
  return min(max(cu[s + 1], seq_begin(cu, s, TB)), TB);
}

template <int DK>
__device__ __forceinline__ void prep_body(char* smem, int64_t blk, const PrepArgs& pa) {
  constexpr int NS = DK / 32;
  using F = Elt<float>;
  const __bf16* __restrict__ const q = pa.q;
  const __bf16* __restrict__ const k = pa.k;
  const float* __restrict__ const gate = pa.gate;
  const float* __restrict__ const beta = pa.beta;
  char* __restrict__ const ws = pa.ws;
  const int gate_logit = pa.gate_logit;
  const float G = pa.G;
  const int B = pa.B, H = pa.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  const int64_t job = blk * kPrepWaves + wave;   // no barriers in this kernel: idle waves return
  int T, b, h, c;
  int64_t tok0;                                  // token (b, 0, h)
  if (pa.cu) {
    // packed sequences: job = h * nslot + slot
    if (job >= (int64_t)H * pa.nslot) return;
    h = (int)(job / pa.nslot);
    const int slot = (int)(job - (int64_t)h * pa.nslot);
    int lo = 0, hi = B - 1;                      // the last s with slot(s, 0) <= slot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seq_begin(pa.cu, mid, pa.TB) / 32 + mid <= slot) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    const int tb = seq_begin(pa.cu, b, pa.TB);
    T = seq_end(pa.cu, b, pa.TB) - tb;
    c = slot - (tb / 32 + b);
    if (c < 0 || c >= ((T + 31) >> 5)) return;   // a slot no pair uses
    tok0 = (int64_t)tb * H + h;
  } else {
    T = pa.T;
    const int NSC = (T + 31) >> 5;
    if (job >= (int64_t)B * H * NSC) return;
    const int head = (int)(job / NSC);
    c = (int)(job - (int64_t)head * NSC);
    b = head / H;
    h = head - b * H;
    tok0 = (int64_t)b * pa.TB * H + h;
  }

  char* scr = smem + wave * (kPrepScr + kPrepRows);
  char* rows = scr + kPrepScr;
  float* sA0 = reinterpret_cast<float*>(scr);
  float* sA1 = reinterpret_cast<float*>(scr + 1024);
  float* sB = reinterpret_cast<float*>(scr + 2048);
  float* sG = reinterpret_cast<float*>(scr + 2176);
  float* sNk = reinterpret_cast<float*>(scr + 2304);
  float* sNq = reinterpret_cast<float*>(scr + 2432);
  char* wr = ws + job * WsRec::BYTES;

  // Loads (rows clamped to T-1: padding tokens need no masking of q or k --
  // with beta = 0 and g = 0 their rows of T are unit vectors and their columns
  // of Tb are zero, so they contribute nothing anywhere).
  // k and q rows are loaded whole (each 16-lane quarter of a load covers one
  // 256-byte row, or two 128-byte rows at d_k = 64; a quarter spanning 16
  // rows would cost the address unit about three times as much) and turned
  // into MFMA fragments through LDS, in the row blocks of rslot.
  constexpr int NL = DK / 16;                    // 1 KB loads per pair and matrix
  bf16x8 kr[NL], qr[NL];
  int lofs[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int f = (64 * i + lane) * 16;           // byte of the pair's 32 x DK block
    const int r = f / (2 * DK), c16 = (f % (2 * DK)) / 16;
    const int t = min(32 * c + r, T - 1);
    const int off = t * H * DK + 8 * c16;         // fits in 32 bits (checked on the host)
    kr[i] = *reinterpret_cast<const bf16x8*>(k + tok0 * DK + off);
    qr[i] = *reinterpret_cast<const bf16x8*>(q + tok0 * DK + off);
    lofs[i] = ((r >> 4) * NS + (c16 >> 2)) * 1024 + 16 * rslot(r & 15, c16 & 3);
  }
  bf16x8 kf[2][NS], qf[2][NS];
  const int o_frag = 16 * rslot(n, grp);
#pragma unroll
  for (int i = 0; i < NL; ++i) *reinterpret_cast<bf16x8*>(rows + lofs[i]) = kr[i];
  wave_fence();
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int s = 0; s < NS; ++s) kf[x][s] = *reinterpret_cast<const bf16x8*>(rows + (x * NS + s) * 1024 + o_frag);
  wave_fence();   // every fragment of k read before q overwrites the block
#pragma unroll
  for (int i = 0; i < NL; ++i) *reinterpret_cast<bf16x8*>(rows + lofs[i]) = qr[i];
  wave_fence();
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[x][s] = *reinterpret_cast<const bf16x8*>(rows + (x * NS + s) * 1024 + o_frag);
  float gx[2], bt[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    const int t = min(32 * c + 16 * x + n, T - 1);
    gx[x] = gate[tok0 + (int64_t)t * H];
    bt[x] = beta[tok0 + (int64_t)t * H];
    if (pa.raw) bt[x] = sigmoid_f(bt[x]);
  }
  if (gate_logit && (pa.gsc || pa.gbi)) {
    const float sc = pa.gsc ? pa.gsc[h] : 1.f, sh = pa.gbi ? pa.gbi[h] : 0.f;
#pragma unroll
    for (int x = 0; x < 2; ++x) gx[x] = fmaf(sc, gx[x], sh);
  }

  const int t0 = 32 * c;
  const bool oka = t0 + n < T, okb = t0 + 16 + n < T;
  // padding tokens past T: g = 0, beta = 0 (an identity step)
  const float gav = oka ? (gate_logit ? bounded_gate(gx[0], G) : gx[0]) : 0.f;
  const float gbv = okb ? (gate_logit ? bounded_gate(gx[1], G) : gx[1]) : 0.f;
  const float ba = oka ? bt[0] : 0.f, bb = okb ? bt[1] : 0.f;
  const float Ga = scan16_dpp(gav);
  const float Ga15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Ga), 15));
  const float Gb = Ga15 + scan16_dpp(gbv);
  const float Gb15 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, Gb), 15));
  if (grp == 0) {
    sB[n] = ba;
    sB[16 + n] = bb;
    sG[n] = Ga;
    sG[16 + n] = Gb;
  }
  const bf16x8* ka = kf[0];
  const bf16x8* kb = kf[1];
  const bf16x8* qa = qf[0];
  const bf16x8* qb = qf[1];
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
  // 1/|k_t| and 1/|q_t| (1 without raw inputs): |k|^2 is the diagonal of
  // K K^T above, |q|^2 that of Q Q^T; lane (n, n / 4) holds entry [n][n]
  {
    float ika = 1.f, ikb = 1.f, iqa = 1.f, iqb = 1.f;
    if (pa.raw) {
      f32x4 qqa = zero4(), qqb = zero4();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        qqa = mma32b(qa[s], qa[s], qqa);
        qqb = mma32b(qb[s], qb[s], qqb);
      }
      auto inv = [](float x) { return x > 0.f ? 1.f / sqrtf(x) : 0.f; };
      const int d = n & 3;
      ika = inv(s00[d]);
      ikb = inv(s11[d]);
      iqa = inv(qqa[d]);
      iqb = inv(qqb[d]);
    }
    if (grp == (n >> 2)) {
      sNk[n] = ika;
      sNk[16 + n] = ikb;
      sNq[n] = iqa;
      sNq[16 + n] = iqb;
    }
  }
  wave_fence();
  if (grp == 0) {
    float* gm = reinterpret_cast<float*>(wr + WsRec::GM);
    float* dl = reinterpret_cast<float*>(wr + WsRec::DL);
    float* gq = reinterpret_cast<float*>(wr + WsRec::GMQ);
    const float ea = __expf(Ga), eb = __expf(Gb);
    const float ika = sNk[n], ikb = sNk[16 + n];
    gm[n] = ea * ika;
    gm[16 + n] = eb * ikb;
    dl[n] = __expf(Gb15 - Ga) * ika;
    dl[16 + n] = __expf(Gb15 - Gb) * ikb;
    gq[n] = ea * sNq[n];
    gq[16 + n] = eb * sNq[16 + n];
    if (n == 0) *reinterpret_cast<float*>(wr + WsRec::GC) = __expf(Gb15);
  }
  const f32x4 Gca = reinterpret_cast<const f32x4*>(sG)[grp];       // G_a at the 4 columns
  const f32x4 Gcb = reinterpret_cast<const f32x4*>(sG)[4 + grp];   // G_b at the 4 columns
  // inverse norms: rows (token n of each tile) and the 4 columns
  const f32x4 Kca = reinterpret_cast<const f32x4*>(sNk)[grp];
  const f32x4 Kcb = reinterpret_cast<const f32x4*>(sNk)[4 + grp];
  const float Kra = sNk[n], Krb = sNk[16 + n], Qra = sNq[n], Qrb = sNq[16 + n];
  f32x4 a00, a11, a10, pp00, pp11, pp10;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int sc = 4 * grp + i;
    const float d00 = __expf(fminf(Ga - Gca[i], 0.f));
    const float d11 = __expf(fminf(Gb - Gcb[i], 0.f));
    const float d10 = __expf(fminf(Gb - Gca[i], 0.f));
    a00[i] = sc < n ? ba * d00 * s00[i] * (Kra * Kca[i]) : 0.f;
    a11[i] = sc < n ? bb * d11 * s11[i] * (Krb * Kcb[i]) : 0.f;
    a10[i] = bb * d10 * s10[i] * (Krb * Kca[i]);
    pp00[i] = sc <= n ? d00 * p00[i] * (Qra * Kca[i]) : 0.f;
    pp11[i] = sc <= n ? d11 * p11[i] * (Qrb * Kcb[i]) : 0.f;
    pp10[i] = d10 * p10[i] * (Qrb * Kca[i]);
  }
  reinterpret_cast<f32x4*>(sA0)[n * 4 + grp] = a00;
  reinterpret_cast<f32x4*>(sA1)[n * 4 + grp] = a11;
  {
    const bf16x4 h00 = hi4(pp00), h10 = hi4(pp10), h11 = hi4(pp11);
    reinterpret_cast<bf16x8*>(wr + WsRec::PF0)[lane] = cat8(h00, lo4(pp00, h00));
    reinterpret_cast<bf16x8*>(wr + WsRec::PF1H)[lane] = cat8(h10, h11);
    reinterpret_cast<bf16x8*>(wr + WsRec::PF1L)[lane] = cat8(lo4(pp10, h10), lo4(pp11, h11));
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
  const bf16x4 h00 = hi4(tb00), h10 = hi4(tb10), h11 = hi4(tb11);
  reinterpret_cast<bf16x8*>(wr + WsRec::TB0)[lane] = cat8(h00, lo4(tb00, h00));
  reinterpret_cast<bf16x8*>(wr + WsRec::TB1H)[lane] = cat8(h10, h11);
  reinterpret_cast<bf16x8*>(wr + WsRec::TB1L)[lane] = cat8(lo4(tb10, h10), lo4(tb11, h11));
}

template <int DK>
__global__ __launch_bounds__(64 * kPrepWaves) void chunk_prep_kernel(PrepArgs pa) {
  __shared__ __attribute__((aligned(16))) char smem[kPrepLDS];
  prep_body<DK>(smem, blockIdx.x, pa);
}

// ============================================================== inter-tile

// SPW d_v slices of 16 columns per workgroup (1, or 2 when one slice per
// workgroup would need more than one round of workgroups: the two slices then
// share the loader's k, q and record traffic).  Waves: chain s = s, output
// s = SPW + s, loader 2 SPW, prefetch 2 SPW + 1.
template <int DK, int SPW>
struct CfgS {
  static constexpr int NBUF = SPW == 1 ? 7 : 6;   // LDS records in the loader's ring
  static constexpr int NT = DK / 16, NS = DK / 32;
  // LDS record of one pair (byte offsets)
  static constexpr int KF = 0;                 // [tile][NS] blocks of k rows, slots as rslot
  static constexpr int QF = KF + 2 * NS * 1024;   // the same for q
  static constexpr int VF = QF + 2 * NS * 1024;   // [SPW][32 tokens][16 columns] bf16
  static constexpr int TB = VF + SPW * 1024;   // TB0 | TB1H | TB1L (workspace bytes 0..3071)
  static constexpr int GD = TB + 3072;         // gamma | delta | Gamma (workspace bytes 6144..6655)
  static constexpr int REC = GD + 512;
  // loads per record: k and q blocks, V, TB, GD
  static constexpr int LPP = 4 * NS + SPW + 3 + 1;
  // chain -> output hand-over per slice, double buffered by pair parity;
  // placed first so that its addresses fit the 16-bit offset field of LDS
  // instructions
  static constexpr int OB_H = 0;               // [NS][64] x 16 B   H (bf16)
  static constexpr int OB_U = NS * 1024;       // [2][64] x 16 B    U_a, U_b (f32)
  static constexpr int OB = OB_U + 2048;
  static constexpr int OFF_OB = 0;             // slice s, parity p at OFF_OB + (2 s + p) OB
  static constexpr int OFF_REC = 2 * SPW * OB;
  static constexpr int OFF_PF = OFF_REC + NBUF * REC;   // landing slot of the prefetch loads
  static constexpr int PF_AHEAD = 8;           // pairs between the chain and the prefetch
  static constexpr int LDS = OFF_PF + 256;
  static constexpr int W_OUT = SPW, W_LOADER = 2 * SPW, W_PREFETCH = 2 * SPW + 1;
  static constexpr int THREADS = 64 * (2 * SPW + 2);   // the kernel's launch bound
  static_assert(REC % 256 == 0 && OB % 16 == 0, "LDS alignment");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert((NBUF - 4) * LPP <= 63, "vmcnt range");
};

__device__ inline void map_block(int n, int NH, int NV, int& head, int& vt) {
  // Workgroups are dealt to the 8 XCDs round robin; numbering the blocks so
  // that block n serves head (8a + n % 8) keeps all d_v slices of a head on
  // one XCD, where they share K, q and the workspace through its L2.
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

// Arguments of the inter-tile work over tokens [0, T) of each sequence (the
// pointers may be advanced to a later token; TB is the full sequence length).
struct StateArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const char* ws;
  const float* h0;
  __bf16* o;
  float* hT;
  int B, T, TB, H, DV;
  const int* cu;     // packed sequences, as in PrepArgs
  int nslot;
  // Transition slices (the segmented form of long sequences): ntr further
  // slices of 16 columns after the DV / 16 value slices carry the state map
  // of the pass applied to h0tr ([B, H, DK, DK]; the identity when null),
  // with v = 0 (read from the zero block zv, 1 KB) and no outputs, and leave
  // the result in htr ([B, H, DK, DK]).  o may be null: no outputs stored.
  int ntr;
  const float* h0tr;
  float* htr;
  const __bf16* zv;
};

// TR: the launch may hold transition slices (sa.ntr > 0); otherwise that
// code is compiled out.
template <int DK, int SPW, bool TR>
__device__ __forceinline__ void state_body(char* smem, int blk, const StateArgs& sa) {
  using C = CfgS<DK, SPW>;
  constexpr int NT = C::NT, NS = C::NS, NBUF = C::NBUF;
  const __bf16* __restrict__ const q = sa.q;
  const __bf16* __restrict__ const k = sa.k;
  const __bf16* __restrict__ const v = sa.v;
  const char* __restrict__ const ws = sa.ws;
  const float* const h0 = sa.h0;
  __bf16* __restrict__ const o = sa.o;
  float* const hT = sa.hT;
  const int B = sa.B, H = sa.H, DV = sa.DV;

  const int NVV = DV / 16;                      // value slices
  const int NV = NVV + (TR ? sa.ntr : 0), NVG = NV / SPW;   // slices, slice groups per head
  int head, vg;
  map_block(blk, B * H, NVG, head, vg);
  const int b = head / H, h = head % H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // the slice of a chain or output wave
  const int vt = vg * SPW + (wave < C::W_OUT ? wave : wave < C::W_LOADER ? wave - C::W_OUT : 0);
  const int v0 = vt * 16;
  const bool tr = TR && vt >= NVV;                        // a transition slice
  const int tcol = 16 * (vt - NVV);                       // its first column of the map
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, grp = lane >> 4;
  int T;
  int64_t tok0;                                          // token (b, 0, h)
  const char* wsh;                                       // record of pair 0
  if (sa.cu) {
    const int tb = seq_begin(sa.cu, b, sa.TB);
    T = seq_end(sa.cu, b, sa.TB) - tb;
    tok0 = (int64_t)tb * H + h;
    wsh = ws + ((int64_t)h * sa.nslot + tb / 32 + b) * WsRec::BYTES;
  } else {
    T = sa.T;
    tok0 = (int64_t)b * sa.TB * H + h;
    wsh = ws + (int64_t)head * ((T + 31) >> 5) * WsRec::BYTES;
  }
  const int NSC = (T + 31) >> 5;                          // pairs of tiles
  if (NSC == 0) {
    // an empty packed sequence: hT = h0 (zeros without h0), by the chain waves
    if (wave < C::W_OUT && tr && sa.htr) {
      const int64_t tbase = ((int64_t)b * H + h) * DK * DK;
      for (int r = 0; r < DK; r += 4) {
        const int64_t e = tbase + (int64_t)(r + grp) * DK + tcol + n;
        sa.htr[e] = sa.h0tr ? sa.h0tr[e] : (r + grp == tcol + n ? 1.f : 0.f);
      }
    } else if (wave < C::W_OUT && !tr && hT) {
      const int64_t sbase = ((int64_t)b * H + h) * DK * DV;
      for (int r = 0; r < DK; r += 4)
        hT[sbase + (int64_t)(r + grp) * DV + v0 + n] = h0 ? h0[sbase + (int64_t)(r + grp) * DV + v0 + n] : 0.f;
    }
    return;
  }
  // Record of pair c.  The byte offset goes through an empty asm so that the
  // compiler keeps one scalar base per pair instead of rewriting every LDS
  // address as its own induction variable.
  auto rec_of = [&](int c) -> char* {
    int rb = __builtin_amdgcn_readfirstlane(C::OFF_REC + (c % NBUF) * C::REC);
    asm volatile("" : "+s"(rb));
    return smem + rb;
  };

  // Barriers: one before pair 0, then one after each pair c = 0 .. NSC-1 and
  // one more that lets the output wave finish the last pair: NSC + 2 in all,
  // executed by every wave.

  if (wave == C::W_PREFETCH) {
    // ---------------------------------------------------------- prefetch
    // Line j of pair p (k rows, then q rows, then v rows, then the workspace
    // record, in 128-byte lines) belongs to slice group j % NVG; each lane
    // loads one word of one of this group's lines into a scratch slot nobody
    // reads.
    const int lk = DK / 64, lv = (DV + 63) / 64;
    const int nk = 32 * lk, nv = 32 * lv, nw = (WsRec::BYTES + 127) / 128;
    const int total = 2 * nk + nv + nw;
    const int rounds = (total + 64 * NVG - 1) / (64 * NVG);
    lds_void* const junk = (lds_void*)(smem + C::OFF_PF);
    auto touch = [&](int p) {
      p = min(p, NSC - 1);
      for (int r = 0; r < rounds; ++r) {
        const int j = vg + NVG * (lane + 64 * r);
        if (j >= total) continue;
        const char* a;
        if (j < 2 * nk) {
          const int jj = j < nk ? j : j - nk;
          const int t = min(32 * p + jj / lk, T - 1);
          a = (const char*)((j < nk ? k : q) + (tok0 + (int64_t)t * H) * DK) + (jj % lk) * 128;
        } else if (j < 2 * nk + nv) {
          const int jj = j - 2 * nk;
          const int t = min(32 * p + jj / lv, T - 1);
          a = (const char*)(v + (tok0 + (int64_t)t * H) * DV) + (jj % lv) * 128;
        } else {
          a = wsh + (int64_t)p * WsRec::BYTES + (j - 2 * nk - nv) * 128;
        }
        __builtin_amdgcn_global_load_lds(a, junk, 4, 0, 0);
      }
    };
#pragma unroll 1
    for (int c = 0; c < C::PF_AHEAD; ++c) touch(c);
    wg_barrier();
#pragma unroll 1
    for (int c = 0; c <= NSC; ++c) {
      touch(c + C::PF_AHEAD);
      wait_vmcnt<48>();            // bound the loads in flight
      wg_barrier();
    }
    wait_vmcnt<0>();               // nothing may land after the workgroup ends
    return;
  }

  if (wave == C::W_LOADER) {
    // ------------------------------------------------------------ loader
    // Ring of NBUF records; pair c lives in record c % NBUF.  During pair c
    // the chain reads records c and c + 1 and the output wave record c - 1,
    // so the record of pair c - 2 is free for pair c + NBUF - 2, and pairs up
    // to c + 2 must have landed by the barrier that ends pair c.  Pair indices
    // are clamped so that every load is valid and the load count never varies.
    // Lane L fills slot L of a block: row L / 4, chunk (L % 4) ^ sw(row).
    const int lrow = lane >> 2, lchunk = (lane & 3) ^ rsw(lane >> 2);
    const __bf16* const kb0 = k + tok0 * DK + 8 * lchunk;
    const __bf16* const qb0 = q + tok0 * DK + 8 * lchunk;
    // a group of transition slices reads its zero v from zv (lane L: bytes
    // 16 L .. 16 L + 15 of the 1 KB block)
    const bool trg = TR && vg * SPW >= NVV;
    const __bf16* const vb0 = v + tok0 * DV + 16 * vg * SPW + 8 * (lane & 1);
    const __bf16* const zvl = sa.zv + 8 * lane;
    auto issue = [&](int c) {
      c = min(c, NSC - 1);
      char* rec = rec_of(c);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int roff = min(32 * c + 16 * x + lrow, T - 1) * H * DK;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          lds_dma16(kb0 + roff + 32 * s, rec + C::KF + (x * NS + s) * 1024);
          lds_dma16(qb0 + roff + 32 * s, rec + C::QF + (x * NS + s) * 1024);
        }
      }
      {  // V of each slice: lane L fetches 8 columns (half L % 2) of token L / 2 of the pair
        const int t = min(32 * c + (lane >> 1), T - 1);
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl)
          lds_dma16(trg ? zvl : vb0 + t * H * DV + 16 * sl, rec + C::VF + sl * 1024);
      }
      const char* wr = wsh + (int64_t)c * WsRec::BYTES + 16 * lane;
#pragma unroll
      for (int i = 0; i < 3; ++i) lds_dma16(wr + i * 1024, rec + C::TB + i * 1024);
      if (lane < 32) lds_dma16(wr + WsRec::GM, rec + C::GD);
    };
    constexpr int kAhead = (NBUF - 4) * C::LPP;   // loads allowed in flight at a barrier
#pragma unroll 1
    for (int c = 0; c < NBUF - 2; ++c) issue(c);
    wait_vmcnt<kAhead>();                          // pairs 0 and 1 landed
    wg_barrier();
#pragma unroll 1
    for (int c = 0; c <= NSC; ++c) {
      issue(c + NBUF - 2);                         // into the record of pair c - 2
      wait_vmcnt<kAhead>();                        // pair c + 2 landed
      wg_barrier();
    }
    wait_vmcnt<0>();
    return;
  }

  if (wave < C::W_OUT) {
    // ------------------------------------------------------------ chain wave
    f32x4 Hacc[NT];
    const int64_t sbase = ((int64_t)b * H + h) * DK * DV;
    const int64_t tbase = ((int64_t)b * H + h) * DK * DK;
    auto srow = [&](int t, int i) { return 32 * (t >> 1) + 8 * grp + 4 * (t & 1) + i; };
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        Hacc[t][i] = !tr ? (h0 ? h0[sbase + (int64_t)srow(t, i) * DV + v0 + n] : 0.f)
                   : sa.h0tr ? sa.h0tr[tbase + (int64_t)srow(t, i) * DK + tcol + n]
                             : (srow(t, i) == tcol + n ? 1.f : 0.f);
    bf16x8 Hb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) Hb[s] = cat8(hi4(Hacc[2 * s]), hi4(Hacc[2 * s + 1]));
    // Per-lane byte offsets inside a record (the record base is added per pair).
    const int o_kf = 16 * rslot(n, grp);                 // K fragment rows
    // transposing read: lane (j, grp) points at K[4 grp + j/4][rho chunk j%4]
    const int o_kt = 16 * rslot(4 * grp + (n >> 2), n & 3);
    const int o_v = C::VF + (vt - vg * SPW) * 1024 + 8 * lane;   // V, transposing read
    const int o_tb = C::TB + 16 * lane;
    const int o_gd = C::GD + 16 * grp;
    char* const obh = smem + C::OFF_OB + 2 * (vt - vg * SPW) * C::OB + C::OB_H + 16 * lane;

    struct Ops { bf16x8 ka[NS], kb[NS]; f32x4 ga, gb, da, db; float Gam; s16x4_t va, vb;
                 bf16x8 tb0, tb1h, tb1l; };
    auto fetch = [&](int c, Ops& x) {
      const char* rec = rec_of(c);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        x.ka[s] = *reinterpret_cast<const bf16x8*>(rec + o_kf + s * 1024);
        x.kb[s] = *reinterpret_cast<const bf16x8*>(rec + o_kf + (NS + s) * 1024);
      }
      // V in accumulator layout: lane (n, grp) receives V[4 grp + r][n], r = 0..3
      x.va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rec + o_v));
      x.vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rec + o_v + 512));
      x.ga = *reinterpret_cast<const f32x4*>(rec + o_gd);
      x.gb = *reinterpret_cast<const f32x4*>(rec + o_gd + 64);
      x.tb0 = *reinterpret_cast<const bf16x8*>(rec + o_tb);
      x.tb1h = *reinterpret_cast<const bf16x8*>(rec + o_tb + 1024);
      x.tb1l = *reinterpret_cast<const bf16x8*>(rec + o_tb + 2048);
      x.da = *reinterpret_cast<const f32x4*>(rec + o_gd + 128);
      x.db = *reinterpret_cast<const f32x4*>(rec + o_gd + 192);
      x.Gam = *reinterpret_cast<const float*>(rec + C::GD + 256);
    };

    // One pair: operands in `cur`, those of the next pair fetched into `nxt`.
    auto pair = [&](int c, const Ops& cur, Ops& nxt) {
      const char* rec = rec_of(c);
      char* ob = obh + (c & 1) * C::OB;
      wait_lgkm0();                // this pair's operands (fetched during the last pair)
      // hand H (bf16, the state before this pair) to the output wave
#pragma unroll
      for (int s = 0; s < NS; ++s) *reinterpret_cast<bf16x8*>(ob + s * 1024) = Hb[s];
      // R = K H, both tiles
      f32x4 Ra = zero4(), Rb = zero4();
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Ra = mma32b(cur.ka[s], Hb[s], Ra);
        Rb = mma32b(cur.kb[s], Hb[s], Rb);
      }
      // K^T fragments of this pair for the state update (transposing reads)
      s16x4_t kta[NT], ktb[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int off = o_kt + (t >> 1) * 1024 + 8 * (t & 1);
        kta[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rec + off));
        ktb[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(rec + off + NS * 1024));
      }
      // operands of the next pair (its record has landed: see the loader)
      fetch(c + 1, nxt);
#pragma unroll
      for (int t = 0; t < NT; ++t) Hacc[t] = Hacc[t] * cur.Gam;
      f32x4 Ya, Yb;
      const bf16x4 va = __builtin_bit_cast(bf16x4, cur.va), vb = __builtin_bit_cast(bf16x4, cur.vb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Ya[i] = (float)va[i] - cur.ga[i] * Ra[i];
        Yb[i] = (float)vb[i] - cur.gb[i] * Rb[i];
      }
      const bf16x4 ya = hi4(Ya), yb = hi4(Yb);
      // U_a = Tb00 Y_a ; U_b = Tb10 Y_a + Tb11 Y_b   (Tb in hi + lo parts)
      const f32x4 Ua = mma32b(cur.tb0, cat8(ya, ya), zero4());
      f32x4 Ub = mma32b(cur.tb1h, cat8(ya, yb), zero4());
      Ub = mma32b(cur.tb1l, cat8(ya, yb), Ub);
      *reinterpret_cast<f32x4*>(ob + C::OB_U) = Ua;
      *reinterpret_cast<f32x4*>(ob + C::OB_U + 1024) = Ub;
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
        const bf16x8 kt = cat8(__builtin_bit_cast(bf16x4, kta[t]), __builtin_bit_cast(bf16x4, ktb[t]));
        Hacc[t] = mma32b(kt, up, Hacc[t]);
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) Hb[s] = cat8(hi4(Hacc[2 * s]), hi4(Hacc[2 * s + 1]));
      wait_lgkm0();                // hand-over written before the barrier
      wg_barrier();
    };

    wg_barrier();                  // pairs 0 and 1 landed
    Ops A, Bo;                     // two operand sets, used in turn
    fetch(0, A);
#pragma unroll 1
    for (int c = 0; c < NSC; c += 2) {
      pair(c, A, Bo);
      if (c + 1 < NSC) pair(c + 1, Bo, A);
    }
    wg_barrier();                  // the output wave's last pair
    if (!tr && hT) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          hT[sbase + (int64_t)srow(t, i) * DV + v0 + n] = Hacc[t][i];
    } else if (tr && sa.htr) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sa.htr[tbase + (int64_t)srow(t, i) * DK + tcol + n] = Hacc[t][i];
    }
    return;
  }

  // -------------------------------------------------------------- output wave
  // Pair c is computed after the barrier that ends the chain's pair c.  Its q
  // fragments come from the pair's record; P and gamma are read straight from
  // global memory (contiguous lines, shared by every d_v slice of the head),
  // kDepth pairs ahead.
  // The products are formed transposed, O^T = H^T Q^T diag(gamma) + U^T P^T
  // (the same fragments with the operands swapped), so that lane (n, grp)
  // ends with columns 4 grp .. 4 grp + 3 of token n: one 8-byte store per tile.
  {
    constexpr int kDepth = 4;
    const bool store_o = o && !tr;
    __bf16* const orow = o + (tok0 + (int64_t)n * H) * DV + v0 + 4 * grp;
    const int ostride = H * DV;
    const char* const obh = smem + C::OFF_OB + 2 * (vt - vg * SPW) * C::OB + C::OB_H + 16 * lane;
    const int o_qf = C::QF + 16 * rslot(n, grp);
    struct Oin { bf16x8 pf0, pf1h, pf1l; float ga, gb; };
    auto gload = [&](Oin& x, int c) {
      c = min(c, NSC - 1);
      const char* wr = wsh + (int64_t)c * WsRec::BYTES;
      x.pf0 = reinterpret_cast<const bf16x8*>(wr + WsRec::PF0)[lane];
      x.pf1h = reinterpret_cast<const bf16x8*>(wr + WsRec::PF1H)[lane];
      x.pf1l = reinterpret_cast<const bf16x8*>(wr + WsRec::PF1L)[lane];
      x.ga = reinterpret_cast<const float*>(wr + WsRec::GMQ)[n];
      x.gb = reinterpret_cast<const float*>(wr + WsRec::GMQ)[16 + n];
    };
    auto pair = [&](Oin& x, int c) {
      const char* ob = obh + (c & 1) * C::OB;
      const char* qf = rec_of(c) + o_qf;
      f32x4 Oa = zero4(), Ob = zero4();   // lane (n, grp) reg i: O[token n][4 grp + i]
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 hb = *reinterpret_cast<const bf16x8*>(ob + s * 1024);
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qf + s * 1024);
        const bf16x8 qb = *reinterpret_cast<const bf16x8*>(qf + (NS + s) * 1024);
        Oa = mma32b(hb, qa, Oa);
        Ob = mma32b(hb, qb, Ob);
      }
      const f32x4 Ua = *reinterpret_cast<const f32x4*>(ob + C::OB_U);
      const f32x4 Ub = *reinterpret_cast<const f32x4*>(ob + C::OB_U + 1024);
      wait_lgkm0();   // hand-over read: the chain may overwrite it after the next barrier
      const bf16x4 uah = hi4(Ua), ubh = hi4(Ub);
      const bf16x4 ual = lo4(Ua, uah), ubl = lo4(Ub, ubh);
      Oa = Oa * x.ga;
      Ob = Ob * x.gb;
      // O_a += P00 U_a ; O_b += P10 U_a + P11 U_b  (P and U in hi + lo parts)
      Oa = mma32b(cat8(uah, uah), x.pf0, Oa);
      Oa = mma32b(cat8(ual, bf16x4{}), x.pf0, Oa);
      Ob = mma32b(cat8(uah, ubh), x.pf1h, Ob);
      Ob = mma32b(cat8(uah, ubh), x.pf1l, Ob);
      Ob = mma32b(cat8(ual, ubl), x.pf1h, Ob);
      __bf16* oc = orow + (int64_t)(32 * c) * ostride;
      if (store_o && 32 * c + n < T) *reinterpret_cast<bf16x4*>(oc) = hi4(Oa);
      if (store_o && 32 * c + 16 + n < T) *reinterpret_cast<bf16x4*>(oc + 16 * ostride) = hi4(Ob);
    };
    Oin s0, s1, s2, s3;
    static_assert(kDepth == 4, "four register sets below");
    gload(s0, 0);
    gload(s1, 1);
    gload(s2, 2);
    gload(s3, 3);
    wg_barrier();    // before pair 0
    wg_barrier();    // after the chain's pair 0
    auto step = [&](Oin& x, int c) {
      pair(x, c);
      gload(x, c + kDepth);
      wg_barrier();
    };
    // Whole groups of kDepth pairs first: every path around the loop then
    // issues the loads in the same order, and the compiler's wait before each
    // pair covers only that pair's loads.
    int c = 0;
#pragma unroll 1
    for (; c + kDepth <= NSC; c += kDepth) {
      step(s0, c);
      step(s1, c + 1);
      step(s2, c + 2);
      step(s3, c + 3);
    }
    if (c < NSC) step(s0, c);
    if (c + 1 < NSC) step(s1, c + 1);
    if (c + 2 < NSC) step(s2, c + 2);
  }
}

// Blocks [0, nstate) carry the state over one stretch of the sequences; any
// blocks after them do the intra-tile work of the next stretch on the compute
// units the state blocks leave idle.  The two share no data within a launch.
template <int DK, int SPW>
__global__ __launch_bounds__(64 * (2 * SPW + 2)) void chunk_state_kernel(
    StateArgs sa, PrepArgs pa, int nstate, int prep_blocks) {
  static_assert(kPrepLDS <= CfgS<DK, SPW>::LDS, "the intra-tile blocks use the same LDS");
  __shared__ __attribute__((aligned(256))) char smem[CfgS<DK, SPW>::LDS];
  if ((int)blockIdx.x < nstate) {
    state_body<DK, SPW, false>(smem, blockIdx.x, sa);
  } else if ((threadIdx.x >> 6) < kPrepWaves) {
    // the intra-tile blocks (their first kPrepWaves waves) each walk the jobs
    // in steps of their number
    const int step = (int)gridDim.x - nstate;
    for (int pb = (int)blockIdx.x - nstate; pb < prep_blocks; pb += step) prep_body<DK>(smem, pb, pa);
  }
}

// The segmented form's launch: blocks [0, nsa) carry the state over a stretch
// of the sequences described by sa, blocks [nsa, nsa + nsb) over one of those
// described by sb (two segments side by side, one slice per workgroup); any
// blocks after them do the intra-tile work of the jobs of pba blocks of pa,
// then pbb of pb.
template <int DK>
__global__ __launch_bounds__(64 * 4) void chunk_state_seg_kernel(
    StateArgs sa, StateArgs sb, int nsa, int nsb, PrepArgs pa, PrepArgs pb, int pba, int pbb) {
  static_assert(kPrepLDS <= CfgS<DK, 1>::LDS, "the intra-tile blocks use the same LDS");
  __shared__ __attribute__((aligned(256))) char smem[CfgS<DK, 1>::LDS];
  const int blk = blockIdx.x;
  if (blk < nsa + nsb) {
    const bool second = blk >= nsa;
    state_body<DK, 1, true>(smem, second ? blk - nsa : blk, second ? sb : sa);
  } else if ((threadIdx.x >> 6) < kPrepWaves) {
    const int step = (int)gridDim.x - nsa - nsb;
    for (int p = blk - nsa - nsb; p < pba + pbb; p += step) {
      const bool second = p >= pba;
      prep_body<DK>(smem, second ? p - pba : p, second ? pb : pa);
    }
  }
}

// Long sequences are cut into stretches of whole pairs.  The intra-tile work
// of stretch 0 runs alone; launch s then carries the state over stretch s
// while its extra blocks prepare stretch s + 1 on the idle compute units.
// The fp32 state passes from one stretch to the next through the workspace
// (read and written in place by the workgroup that owns each slice), so the
// results are those of a single pass: the state crosses the cut exactly.
// Sequences of kStretchAreaPairs pairs or more may be cut (the workspace then
// holds the carried state); stretches have at least kStretchMinPairs pairs,
// and there are at most kMaxStretches (at 64K x 16 heads, 2048 pairs: 4
// stretches 1.22 ms, 8 1.19, 16 1.13, 32 1.21 per call).
constexpr int kStretchAreaPairs = 512;
constexpr int kStretchMinPairs = 128;
constexpr int kMaxStretches = 16;
// Intra-tile blocks launched beside the state blocks: enough to finish the
// next stretch's records within the current stretch (they loop over the jobs),
// few enough not to slow the state blocks down (2 per sequence-head measured
// best at 64K x 16 heads with 16 stretches; launching one block per job slowed
// the state blocks by ~10 %).  Preparing raw q and k costs more per job (the
// Q Q^T chains and the folded norms): 3 per head keep its records on time
// (2 per head: 1.22 ms per call, 3: 1.13, as for prepared inputs).
constexpr int kPrepResidentPerHead = 2;
constexpr int kPrepResidentPerHeadRaw = 3;
constexpr int kPrepResidentMin = 16;

static bool stretch_area(int NSC) { return NSC >= kStretchAreaPairs; }


// ---------------------------------------------------- segmented long sequences
// With few heads the state workgroups leave most compute units idle and the
// serial length T / 32 pairs sets the time.  Long sequences are then cut into
// three segments of pairs, and since the state map of a pair is affine,
// H_out = M H_in + C, the middle segment's map can be formed before its
// start state is known: pass A carries segment 0 from h0 and, side by side,
// segment 1 from zero together with DK / 16 transition slices that carry M
// (the identity stepped with v = 0); a combine step forms segment 2's start
// state M_1 H_1 + C_1; pass B carries segments 1 and 2 from their true start
// states and writes their outputs.  The serial length drops to about 2 T / 3
// pairs.  Each pass runs in stretches with the next stretch's intra-tile work
// beside it, as the one-segment form does.
constexpr int kSegAreaPairs = 3 * kStretchAreaPairs;

static bool seg_area(int NSC) { return NSC >= kSegAreaPairs; }

// out = A Hs + Bv per (sequence, head): A [DK, DK], Hs, Bv, out [DK, DV]
// float32.  One block per (sequence-head, 16 columns); thread: one row,
// 16 / (256 / DK) columns.
template <int DK>
__global__ __launch_bounds__(256) void seg_combine_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ Hs,
                                                          const float* __restrict__ Bv,
                                                          float* __restrict__ out, int DV) {
  constexpr int TPR = 256 / DK, CPT = 16 / TPR;
  const int NVs = DV / 16;
  const int64_t bh = blockIdx.x / NVs;
  const int cs = (int)(blockIdx.x - bh * NVs);
  const int r = threadIdx.x / TPR, c0 = 16 * cs + (threadIdx.x % TPR) * CPT;
  const float* __restrict__ a = A + (bh * DK + r) * DK;
  const float* __restrict__ hs = Hs + bh * DK * DV + c0;
  float acc[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = Bv[(bh * DK + r) * DV + c0 + j];
  for (int kk = 0; kk < DK; ++kk) {
    const float av = a[kk];
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = fmaf(av, hs[(int64_t)kk * DV + j], acc[j]);
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) out[(bh * DK + r) * DV + c0 + j] = acc[j];
}

__global__ void zero_block_kernel(uint4* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = uint4{0u, 0u, 0u, 0u};
}

// Workspace of the segmented form after the records: float32 carry0, carry1,
// hs1, c1, hs2 [B, H, DK, Dv] each, carryT, m1 [B, H, DK, DK] each, then the
// 1 KB zero block.
template <int DK>
static hipError_t launch_pair_seg_t(const void* q, const void* k, const void* v,
                                    const float* gate, int gate_logit, float G, const float* beta,
                                    const float* h0, void* o, float* hT, int B, int T, int H,
                                    int Dv, int raw, void* ws, hipStream_t st, const float* gsc,
                                    const float* gbi) {
  const int NSC = (T + 31) / 32;
  const int cus = device_cus();
  const int NV = Dv / 16, NTR = DK / 16;
  const int nst0 = B * H * NV, nst1 = B * H * (NV + NTR);
  const int P[4] = {0, NSC / 3, 2 * (NSC / 3), NSC};
  const int S = min(kMaxStretches, max(1, (P[1] - P[0]) / kStretchMinPairs));
  char* const wsb = static_cast<char*>(ws);
  const int64_t nst = (int64_t)B * H * DK * Dv, ntt = (int64_t)B * H * DK * DK;
  float* const carry0 = reinterpret_cast<float*>(wsb + (int64_t)B * H * NSC * WsRec::BYTES);
  float* const carry1 = carry0 + nst;
  float* const hs1 = carry1 + nst;
  float* const c1 = hs1 + nst;
  float* const hs2 = c1 + nst;
  float* const carryT = hs2 + nst;
  float* const m1 = carryT + ntt;
  __bf16* const zv = reinterpret_cast<__bf16*>(m1 + ntt);
  // pairs [p0, p1) of stretch s of segment g
  auto span = [&](int g, int s, int& p0, int& p1) {
    const int len = P[g + 1] - P[g];
    p0 = P[g] + (int)((int64_t)len * s / S);
    p1 = P[g] + (int)((int64_t)len * (s + 1) / S);
  };
  auto prep_args = [&](int g, int s) {
    int p0, p1;
    span(g, s, p0, p1);
    const int64_t t0 = 32 * (int64_t)p0;
    PrepArgs a{(const __bf16*)q + t0 * H * DK, (const __bf16*)k + t0 * H * DK,
               gate + t0 * H, beta + t0 * H, wsb + (int64_t)B * H * p0 * WsRec::BYTES,
               gate_logit, G, B, min(32 * p1, T) - 32 * p0, T, H, raw};
    a.gsc = gsc;
    a.gbi = gbi;
    return a;
  };
  auto prep_blocks = [&](int g, int s) {
    int p0, p1;
    span(g, s, p0, p1);
    return (int)(((int64_t)B * H * (p1 - p0) + kPrepWaves - 1) / kPrepWaves);
  };
  auto state_args = [&](int g, int s, const float* hin, float* hout, bool out, int ntr,
                        const float* tin, float* tout) {
    int p0, p1;
    span(g, s, p0, p1);
    const int64_t t0 = 32 * (int64_t)p0;
    StateArgs a{(const __bf16*)q + t0 * H * DK, (const __bf16*)k + t0 * H * DK,
                (const __bf16*)v + t0 * H * Dv, wsb + (int64_t)B * H * p0 * WsRec::BYTES, hin,
                out ? (__bf16*)o + t0 * H * Dv : nullptr, hout, B, min(32 * p1, T) - 32 * p0, T,
                H, Dv};
    a.ntr = ntr;
    a.h0tr = tin;
    a.htr = tout;
    a.zv = zv;
    return a;
  };
  constexpr int kThreads = CfgS<DK, 1>::THREADS;
  auto launch = [&](const StateArgs& sa, const StateArgs& sb, int nsa, int nsb,
                    const PrepArgs& pa, const PrepArgs& pb, int pba, int pbb) {
    const int idle = cus - nsa - nsb;
    const int resident = pba + pbb > 0 ? max(1, min(idle, pba + pbb)) : 0;
    hipLaunchKernelGGL((chunk_state_seg_kernel<DK>), dim3(nsa + nsb + resident), dim3(kThreads),
                       0, st, sa, sb, nsa, nsb, pa, pb, pba, pbb);
    return hipGetLastError();
  };
  hipLaunchKernelGGL(zero_block_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<uint4*>(zv), 64);
  for (int g = 0; g < 2; ++g) {
    hipLaunchKernelGGL((chunk_prep_kernel<DK>), dim3((unsigned)prep_blocks(g, 0)),
                       dim3(64 * kPrepWaves), 0, st, prep_args(g, 0));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // pass A: segment 0 from h0, segment 1 from zero with its state map
  for (int s = 0; s < S; ++s) {
    const bool last = s == S - 1;
    const StateArgs sa = state_args(0, s, s == 0 ? h0 : carry0, last ? hs1 : carry0, true, 0,
                                    nullptr, nullptr);
    const StateArgs sb = state_args(1, s, s == 0 ? nullptr : carry1, last ? c1 : carry1, false,
                                    NTR, s == 0 ? nullptr : carryT, last ? m1 : carryT);
    if (!last)
      e = launch(sa, sb, nst0, nst1, prep_args(0, s + 1), prep_args(1, s + 1),
                 prep_blocks(0, s + 1), prep_blocks(1, s + 1));
    else   // beside the last stretch: segment 2's first stretch
      e = launch(sa, sb, nst0, nst1, prep_args(2, 0), PrepArgs{}, prep_blocks(2, 0), 0);
    if (e != hipSuccess) return e;
  }
  // segment 2's start state
  hipLaunchKernelGGL((seg_combine_kernel<DK>), dim3(B * H * NV), dim3(256), 0, st,
                     (const float*)m1, (const float*)hs1, (const float*)c1, hs2, Dv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // pass B: segments 1 and 2 from their start states, with outputs
  for (int s = 0; s < S; ++s) {
    const bool last = s == S - 1;
    const StateArgs sa = state_args(1, s, s == 0 ? hs1 : carry0, last ? nullptr : carry0, true,
                                    0, nullptr, nullptr);
    const StateArgs sb = state_args(2, s, s == 0 ? hs2 : carry1, last ? hT : carry1, true, 0,
                                    nullptr, nullptr);
    if (!last)
      e = launch(sa, sb, nst0, nst0, prep_args(2, s + 1), PrepArgs{}, prep_blocks(2, s + 1), 0);
    else
      e = launch(sa, sb, nst0, nst0, PrepArgs{}, PrepArgs{}, 0, 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DK>
static hipError_t launch_pair_t(const void* q, const void* k, const void* v, const float* gate,
                                int gate_logit, float G, const float* beta, const float* h0,
                                void* o, float* hT, int B, int T, int H, int Dv, int raw, void* ws,
                                hipStream_t st, const float* gsc, const float* gbi) {
  const int NSC = (T + 31) / 32;
  const int cus = device_cus();
  // two slices per workgroup when one per workgroup would take more than one
  // round of workgroups (one fits per compute unit)
  const int NV = Dv / 16;
  const int spw = (NV % 2 == 0 && (int64_t)B * H * NV > cus) ? 2 : 1;
  const int nstate = B * H * (NV / spw);
  if (seg_area(NSC) && spw == 1 && B * H * (2 * NV + DK / 16) <= cus - 16)
    return launch_pair_seg_t<DK>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, raw,
                                 ws, st, gsc, gbi);
  int S = 1;
  if (stretch_area(NSC) && 2 * nstate <= cus) S = min(kMaxStretches, NSC / kStretchMinPairs);
  const int per_head = raw ? kPrepResidentPerHeadRaw : kPrepResidentPerHead;
  const int resident_cap = min(cus - nstate, max(kPrepResidentMin, per_head * B * H));
  char* const wsb = static_cast<char*>(ws);
  float* const carry = reinterpret_cast<float*>(wsb + (int64_t)B * H * NSC * WsRec::BYTES);
  auto span = [&](int s, int& p0, int& p1) {
    p0 = (int)((int64_t)NSC * s / S);
    p1 = (int)((int64_t)NSC * (s + 1) / S);
  };
  auto prep_args = [&](int s) {
    int p0, p1;
    span(s, p0, p1);
    const int64_t t0 = 32 * (int64_t)p0;
    const int Ts = min(32 * p1, T) - 32 * p0;
    PrepArgs a{(const __bf16*)q + t0 * H * DK, (const __bf16*)k + t0 * H * DK,
               gate + t0 * H, beta + t0 * H, wsb + (int64_t)B * H * p0 * WsRec::BYTES,
               gate_logit, G, B, Ts, T, H, raw};
    a.gsc = gsc;
    a.gbi = gbi;
    return a;
  };
  auto prep_blocks = [&](int s) {
    int p0, p1;
    span(s, p0, p1);
    return (int)(((int64_t)B * H * (p1 - p0) + kPrepWaves - 1) / kPrepWaves);
  };
  {
    const PrepArgs pa = prep_args(0);
    hipLaunchKernelGGL((chunk_prep_kernel<DK>), dim3((unsigned)prep_blocks(0)),
                       dim3(64 * kPrepWaves), 0, st, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int s = 0; s < S; ++s) {
    int p0, p1;
    span(s, p0, p1);
    const int64_t t0 = 32 * (int64_t)p0;
    const StateArgs sa{(const __bf16*)q + t0 * H * DK, (const __bf16*)k + t0 * H * DK,
                       (const __bf16*)v + t0 * H * Dv, wsb + (int64_t)B * H * p0 * WsRec::BYTES,
                       s == 0 ? h0 : carry, (__bf16*)o + t0 * H * Dv, s == S - 1 ? hT : carry,
                       B, min(32 * p1, T) - 32 * p0, T, H, Dv};
    const bool more = s + 1 < S;
    const PrepArgs pa = more ? prep_args(s + 1) : PrepArgs{};
    const int pblocks = more ? prep_blocks(s + 1) : 0;
    const int resident = more ? min(pblocks, max(1, resident_cap)) : 0;
    constexpr int kThreads1 = CfgS<DK, 1>::THREADS, kThreads2 = CfgS<DK, 2>::THREADS;
    if (spw == 2)
      hipLaunchKernelGGL((chunk_state_kernel<DK, 2>), dim3(nstate + resident), dim3(kThreads2), 0,
                         st, sa, pa, nstate, pblocks);
    else
      hipLaunchKernelGGL((chunk_state_kernel<DK, 1>), dim3(nstate + resident), dim3(kThreads1), 0,
                         st, sa, pa, nstate, pblocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

long long chunk_pair_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
  const int NSC = (T + 31) / 32;
  long long n = (long long)B * H * NSC * WsRec::BYTES;
  if (stretch_area(NSC)) n += (long long)B * H * Dk * Dv * 4;
  // the segmented form's further states, state maps and zero block
  if (seg_area(NSC)) n += (long long)B * H * (4LL * Dk * Dv + 2LL * Dk * Dk) * 4 + 1024;
  return n;
}

// Packed sequences: one intra-tile launch over every record slot (idle slots
// return at once), then one inter-tile launch over (sequence, head, slices).
static int varlen_slots(int T, int nseq) { return T / 32 + nseq + 1; }

template <int DK>
static hipError_t launch_varlen_t(const void* q, const void* k, const void* v, const float* gate,
                                  int gate_logit, float G, const float* beta, const float* h0,
                                  void* o, float* hT, const int* cu, int nseq, int T, int H, int Dv,
                                  int raw, void* ws, hipStream_t st, const float* gsc,
                                  const float* gbi) {
  const int nslot = varlen_slots(T, nseq);
  const int NV = Dv / 16;
  const int spw = (NV % 2 == 0 && (int64_t)nseq * H * NV > device_cus()) ? 2 : 1;
  const int nstate = nseq * H * (NV / spw);
  char* const wsb = static_cast<char*>(ws);
  const PrepArgs pa{(const __bf16*)q, (const __bf16*)k, gate, beta, wsb, gate_logit, G,
                    nseq, 0, T, H, raw, cu, nslot, gsc, gbi};
  const int64_t pblocks = ((int64_t)H * nslot + kPrepWaves - 1) / kPrepWaves;
  hipLaunchKernelGGL((chunk_prep_kernel<DK>), dim3((unsigned)pblocks), dim3(64 * kPrepWaves), 0,
                     st, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const StateArgs sa{(const __bf16*)q, (const __bf16*)k, (const __bf16*)v, wsb, h0, (__bf16*)o,
                     hT, nseq, 0, T, H, Dv, cu, nslot};
  constexpr int kThreads1 = CfgS<DK, 1>::THREADS, kThreads2 = CfgS<DK, 2>::THREADS;
  if (spw == 2)
    hipLaunchKernelGGL((chunk_state_kernel<DK, 2>), dim3(nstate), dim3(kThreads2), 0, st, sa,
                       PrepArgs{}, nstate, 0);
  else
    hipLaunchKernelGGL((chunk_state_kernel<DK, 1>), dim3(nstate), dim3(kThreads1), 0, st, sa,
                       PrepArgs{}, nstate, 0);
  return hipGetLastError();
}

long long chunk_pair_varlen_workspace_bytes(int T, int nseq, int H) {
  return (long long)H * varlen_slots(T, nseq) * WsRec::BYTES;
}

hipError_t launch_chunk_fwd_pair_varlen(const void* q, const void* k, const void* v,
                                        const float* gate, int gate_logit, float G,
                                        const float* beta, const float* h0, void* o, float* hT,
                                        const int* cu, int nseq, int T, int H, int Dk, int Dv,
                                        int raw, void* ws, hipStream_t st, const float* gsc,
                                        const float* gbi) {
  if (Dk == 64) return launch_varlen_t<64>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, cu, nseq, T, H, Dv, raw, ws, st, gsc, gbi);
  if (Dk == 128) return launch_varlen_t<128>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, cu, nseq, T, H, Dv, raw, ws, st, gsc, gbi);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd_pair(const void* q, const void* k, const void* v, const float* gate,
                                 int gate_logit, float G, const float* beta, const float* h0,
                                 void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                                 int raw, void* ws, hipStream_t st, const float* gsc,
                                 const float* gbi) {
  if (Dk == 64) return launch_pair_t<64>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, raw, ws, st, gsc, gbi);
  if (Dk == 128) return launch_pair_t<128>(q, k, v, gate, gate_logit, G, beta, h0, o, hT, B, T, H, Dv, raw, ws, st, gsc, gbi);
  return hipErrorInvalidValue;
}

}  // namespace la
