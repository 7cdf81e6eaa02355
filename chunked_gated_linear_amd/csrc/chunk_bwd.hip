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
//   bwd_hstates_kernel  per (sequence, head, 16 columns of d_v), serial over
//                       tiles: the state at every tile start;
//   bwd_dh_kernel       same split, serial backwards: dH' at every tile end,
//                       and dh0;
//   bwd_grad_kernel     per tile, all of d_v: dq, dk, dv, dbeta, dg.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "la_device.h"
#include "la_launch.h"

namespace la {
namespace {

constexpr int kT = 16;          // tokens per tile
constexpr int kBwdThreads = 256;

// Record of one tile (floats).
struct BRec {
  static constexpr int TINV = 0;     // (I + A)^-1, row-major 16 x 16
  static constexpr int P = 256;      // E o Q K^T, lower incl. diagonal
  static constexpr int EKK = 512;    // E o K K^T, strictly lower
  static constexpr int G = 768;      // in-tile running sum of g
  static constexpr int BETA = 784;
  static constexpr int FLOATS = 800;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* gate;
  const float* beta;
  const float* h0;
  const float* dhT;
  float* dq;
  float* dk;
  float* dv;
  float* dgate;
  float* dbeta;
  float* dh0;
  float* rec;
  float* hs;    // [B, H, NT, Dk, Dv] state at each tile start
  float* dhs;   // [B, H, NT, Dk, Dv] gradient of each tile's end state
  int gate_logit;
  float G;
  int B, T, H, Dv, NT;
};

// Eight consecutive elements as fp32 (16-byte aligned source).
template <typename E> struct Ld8;
template <> struct Ld8<__bf16> {
  __device__ static inline void run(const __bf16* p, float* o) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Ld8<float> {
  __device__ static inline void run(const float* p, float* o) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

template <typename E> __device__ inline float ld1(const E* p) { return (float)*p; }

// Rows of one tile of a [B, T, H, D] tensor into LDS (fp32, row pitch D + 1),
// zeros past the end of the sequence.
template <typename E, int D>
__device__ inline void load_tile(float (*dst)[D + 1], const E* src, int b, int c, int h,
                                 const BwdArgs& a) {
  constexpr int PER_ROW = D / 8;
  for (int x = threadIdx.x; x < kT * PER_ROW; x += kBwdThreads) {
    const int t = x / PER_ROW, c8 = (x % PER_ROW) * 8;
    const int tok = c * kT + t;
    float f[8];
    if (tok < a.T) {
      Ld8<E>::run(src + (((int64_t)b * a.T + tok) * a.H + h) * D + c8, f);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[t][c8 + i] = f[i];
  }
}

// The same tile rows in two steps: fetch() issues this thread's share of the
// loads (8 consecutive elements of one row; threads beyond the tile's
// 16 * D / 8 pieces hold nothing), put() stores them into LDS.  Splitting the
// two lets a serial loop issue tile c + 1's loads before working on tile c.
template <typename E, int D>
struct TilePiece {
  float f[8];
  __device__ inline void fetch(const E* src, int b, int c, int h, const BwdArgs& a) {
    constexpr int PER_ROW = D / 8;
    static_assert(kT * PER_ROW <= kBwdThreads, "one piece per thread");
    const int x = threadIdx.x;
    const int tok = c * kT + x / PER_ROW;
    if (x < kT * PER_ROW && tok < a.T) {
      Ld8<E>::run(src + (((int64_t)b * a.T + tok) * a.H + h) * D + (x % PER_ROW) * 8, f);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = 0.f;
    }
  }
  __device__ inline void put(float (*dst)[D + 1]) const {
    constexpr int PER_ROW = D / 8;
    const int x = threadIdx.x;
    if (x < kT * PER_ROW) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dst[x / PER_ROW][(x % PER_ROW) * 8 + i] = f[i];
    }
  }
};

// A tile's per-token scalars from its record, fetched ahead: g and beta for
// threads < 16, the tile's total decay sum for all.
struct TileScalars {
  float g, bt, gC;
  __device__ inline void fetch(const float* rec) {
    const int tid = threadIdx.x;
    g = tid < kT ? rec[BRec::G + tid] : 0.f;
    bt = tid < kT ? rec[BRec::BETA + tid] : 0.f;
    gC = rec[BRec::G + kT - 1];
  }
  // the values load_scalars would produce
  __device__ inline void put(float* sG, float* sB, float* sGam, float* sEc, float& gamC) const {
    const int tid = threadIdx.x;
    if (tid < kT) {
      sG[tid] = g;
      sB[tid] = bt;
      sGam[tid] = __expf(g);
      sEc[tid] = __expf(gC - g);
    }
    gamC = __expf(gC);
  }
};

__device__ inline float gate_at(const BwdArgs& a, int64_t idx) {
  const float x = a.gate[idx];
  return a.gate_logit ? bounded_gate(x, a.G) : x;
}

// ---------------------------------------------------------------- tile prep
template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(BwdArgs a) {
  __shared__ float sK[kT][DK + 1], sQ[kT][DK + 1];
  __shared__ float sG[kT], sB[kT];
  __shared__ float sA[kT][kT + 1], sTi[kT][kT + 1];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int c = (int)(tile % a.NT);
  const int64_t bh = tile / a.NT;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  load_tile<E, DK>(sK, static_cast<const E*>(a.k), b, c, h, a);
  load_tile<E, DK>(sQ, static_cast<const E*>(a.q), b, c, h, a);
  if (tid < kT) {
    const int tok = c * kT + tid;
    const int64_t idx = ((int64_t)b * a.T + tok) * a.H + h;
    sG[tid] = tok < a.T ? gate_at(a, idx) : 0.f;
    sB[tid] = tok < a.T ? a.beta[idx] : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    float acc = 0.f;
    for (int t = 0; t < kT; ++t) {
      acc += sG[t];
      sG[t] = acc;
    }
  }
  __syncthreads();
  const int t = tid >> 4, i = tid & 15;
  float kk = 0.f, qk = 0.f;
#pragma unroll 8
  for (int r = 0; r < DK; ++r) {
    kk += sK[t][r] * sK[i][r];
    qk += sQ[t][r] * sK[i][r];
  }
  const float e = i <= t ? __expf(sG[t] - sG[i]) : 0.f;
  const float ekk = i < t ? e * kk : 0.f;
  float* rec = a.rec + tile * BRec::FLOATS;
  rec[BRec::EKK + tid] = ekk;
  rec[BRec::P + tid] = e * qk;
  sA[t][i] = sB[t] * ekk;
  __syncthreads();
  // (I + A) T = I, row by row: T[r][j] = [r == j] - sum_{m < r} A[r][m] T[m][j]
  for (int r = 0; r < kT; ++r) {
    if (tid < kT) {
      float s = r == tid ? 1.f : 0.f;
      for (int m = 0; m < r; ++m) s -= sA[r][m] * sTi[m][tid];
      sTi[r][tid] = s;
    }
    __syncthreads();
  }
  rec[BRec::TINV + tid] = sTi[t][i];
  if (tid < kT) {
    rec[BRec::G + tid] = sG[tid];
    rec[BRec::BETA + tid] = sB[tid];
  }
}

// Per-tile scalars shared by the serial kernels, from the record.
__device__ inline void load_scalars(const float* rec, float* sG, float* sB, float* sGam,
                                    float* sEc, float& gamC) {
  const int tid = threadIdx.x;
  if (tid < kT) {
    const float g = rec[BRec::G + tid];
    const float gC = rec[BRec::G + kT - 1];
    sG[tid] = g;
    sB[tid] = rec[BRec::BETA + tid];
    sGam[tid] = __expf(g);
    sEc[tid] = __expf(gC - g);
  }
  gamC = __expf(rec[BRec::G + kT - 1]);
}

// ------------------------------------------------- states at every tile start
template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads) void bwd_hstates_kernel(BwdArgs a) {
  constexpr int TPR = kBwdThreads / DK;   // threads per state row
  constexpr int CPT = 16 / TPR;           // columns per thread
  __shared__ float sK[kT][DK + 1];
  __shared__ float sH[DK][17];
  __shared__ float sY[kT][17], sU[kT][17];
  __shared__ float sTi[kT][kT + 1];
  __shared__ float sG[kT], sB[kT], sGam[kT], sEc[kT];
  const int tid = threadIdx.x;
  const int NV = a.Dv / 16;
  const int sl = (int)(blockIdx.x % NV);
  const int64_t bh = blockIdx.x / NV;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int r = tid / TPR, j0 = (tid % TPR) * CPT;
  const int t = tid >> 4, j = tid & 15;
  const int col = 16 * sl;
  float Hr[CPT];
#pragma unroll
  for (int x = 0; x < CPT; ++x)
    Hr[x] = a.h0 ? a.h0[(bh * DK + r) * a.Dv + col + j0 + x] : 0.f;
  const E* vp = static_cast<const E*>(a.v);
  const E* kp = static_cast<const E*>(a.k);
  // tile c's loads, issued during tile c - 1
  TilePiece<E, DK> nk;
  TileScalars ns;
  float ntinv, nv;
  auto fetch = [&](int c) {
    const float* rec = a.rec + (bh * a.NT + c) * BRec::FLOATS;
    nk.fetch(kp, b, c, h, a);
    ns.fetch(rec);
    ntinv = rec[BRec::TINV + tid];
    const int tok = c * kT + t;
    nv = tok < a.T ? ld1(vp + (((int64_t)b * a.T + tok) * a.H + h) * a.Dv + col + j) : 0.f;
  };
  fetch(0);
  for (int c = 0; c < a.NT; ++c) {
    float* hsp = a.hs + ((bh * a.NT + c) * DK + r) * a.Dv + col + j0;
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      hsp[x] = Hr[x];
      sH[r][j0 + x] = Hr[x];
    }
    nk.put(sK);
    sTi[t][j] = ntinv;
    float gamC;
    ns.put(sG, sB, sGam, sEc, gamC);
    const float vv = nv;
    if (c + 1 < a.NT) fetch(c + 1);
    __syncthreads();
    float R = 0.f;
#pragma unroll 8
    for (int rr = 0; rr < DK; ++rr) R += sK[t][rr] * sH[rr][j];
    sY[t][j] = sB[t] * (vv - sGam[t] * R);
    __syncthreads();
    float U = 0.f;
    for (int i = 0; i <= t; ++i) U += sTi[t][i] * sY[i][j];
    sU[t][j] = U;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      float acc = gamC * Hr[x];
      for (int i = 0; i < kT; ++i) acc += sEc[i] * sK[i][r] * sU[i][j0 + x];
      Hr[x] = acc;
    }
    __syncthreads();
  }
}

// ------------------------------------- gradients of every tile's end state
template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads) void bwd_dh_kernel(BwdArgs a) {
  constexpr int TPR = kBwdThreads / DK;
  constexpr int CPT = 16 / TPR;
  __shared__ float sK[kT][DK + 1], sQ[kT][DK + 1];
  __shared__ float sD[DK][17];
  __shared__ float sDO[kT][17], sDU[kT][17], sZ[kT][17], sOg[kT][17];
  __shared__ float sTi[kT][kT + 1], sP[kT][kT + 1];
  __shared__ float sG[kT], sB[kT], sGam[kT], sEc[kT];
  const int tid = threadIdx.x;
  const int NV = a.Dv / 16;
  const int sl = (int)(blockIdx.x % NV);
  const int64_t bh = blockIdx.x / NV;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int r = tid / TPR, j0 = (tid % TPR) * CPT;
  const int t = tid >> 4, j = tid & 15;
  const int col = 16 * sl;
  float D[CPT];
#pragma unroll
  for (int x = 0; x < CPT; ++x)
    D[x] = a.dhT ? a.dhT[(bh * DK + r) * a.Dv + col + j0 + x] : 0.f;
  const E* dop = static_cast<const E*>(a.dout);
  const E* kp = static_cast<const E*>(a.k);
  const E* qp = static_cast<const E*>(a.q);
  // tile c's loads, issued during tile c + 1
  TilePiece<E, DK> nk, nq;
  TileScalars ns;
  float ntinv, np, ndo;
  auto fetch = [&](int c) {
    const float* rec = a.rec + (bh * a.NT + c) * BRec::FLOATS;
    nk.fetch(kp, b, c, h, a);
    nq.fetch(qp, b, c, h, a);
    ns.fetch(rec);
    ntinv = rec[BRec::TINV + tid];
    np = rec[BRec::P + tid];
    const int tok = c * kT + t;
    ndo = tok < a.T ? ld1(dop + (((int64_t)b * a.T + tok) * a.H + h) * a.Dv + col + j) : 0.f;
  };
  if (a.NT > 0) fetch(a.NT - 1);
  for (int c = a.NT - 1; c >= 0; --c) {
    float* dsp = a.dhs + ((bh * a.NT + c) * DK + r) * a.Dv + col + j0;
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      dsp[x] = D[x];
      sD[r][j0 + x] = D[x];
    }
    nk.put(sK);
    nq.put(sQ);
    sTi[t][j] = ntinv;
    sP[t][j] = np;
    float gamC;
    ns.put(sG, sB, sGam, sEc, gamC);
    sDO[t][j] = ndo;
    if (c > 0) fetch(c - 1);
    __syncthreads();
    float KdH = 0.f;
#pragma unroll 8
    for (int rr = 0; rr < DK; ++rr) KdH += sK[t][rr] * sD[rr][j];
    float dU = sEc[t] * KdH;
    for (int s = t; s < kT; ++s) dU += sP[s][t] * sDO[s][j];
    sDU[t][j] = dU;
    sOg[t][j] = sGam[t] * sDO[t][j];
    __syncthreads();
    float dY = 0.f;
    for (int s = t; s < kT; ++s) dY += sTi[s][t] * sDU[s][j];
    sZ[t][j] = sB[t] * sGam[t] * dY;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < CPT; ++x) {
      float acc = gamC * D[x];
      for (int s = 0; s < kT; ++s) acc += sQ[s][r] * sOg[s][j0 + x] - sK[s][r] * sZ[s][j0 + x];
      D[x] = acc;
    }
    __syncthreads();
  }
  if (a.dh0) {
#pragma unroll
    for (int x = 0; x < CPT; ++x) a.dh0[(bh * DK + r) * a.Dv + col + j0 + x] = D[x];
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

template <typename E, int DK>
__global__ __launch_bounds__(kBwdThreads) void bwd_grad_kernel(BwdArgs a) {
  constexpr int RB = DK / 16;   // rows of dq / dk per thread
  __shared__ float sK[kT][DK + 1], sQ[kT][DK + 1];
  __shared__ float sH[DK][17], sD[DK][17];
  __shared__ float sV[kT][17], sDO[kT][17], sY[kT][17], sU[kT][17], sDU[kT][17], sDY[kT][17];
  __shared__ float sTi[kT][kT + 1], sP[kT][kT + 1];
  __shared__ float sPE[kT][kT + 1], sM[kT][kT + 1], sPP[kT][kT + 1], sAA[kT][kT + 1];
  __shared__ float sG[kT], sB[kT], sGam[kT], sEc[kT];
  __shared__ float sRowB[kT], sRowG[kT], sRowW[kT], sRowAK[kT];
  __shared__ float sHdH[kBwdThreads / 64];
  const int tid = threadIdx.x;
  const int64_t tile = blockIdx.x;
  const int c = (int)(tile % a.NT);
  const int64_t bh = tile / a.NT;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int t = tid >> 4, j = tid & 15;        // (token, column) or (token, token)
  // dq / dk rows of this thread: j, j + 16, ..., so the 16 threads of a token
  // read 16 different LDS banks of a state slice and store 16 adjacent floats
  const float* rec = a.rec + tile * BRec::FLOATS;
  load_tile<E, DK>(sK, static_cast<const E*>(a.k), b, c, h, a);
  load_tile<E, DK>(sQ, static_cast<const E*>(a.q), b, c, h, a);
  sTi[t][j] = rec[BRec::TINV + tid];
  sP[t][j] = rec[BRec::P + tid];
  const float ekk = rec[BRec::EKK + tid];
  float gamC;
  load_scalars(rec, sG, sB, sGam, sEc, gamC);
  const int tok = c * kT + t;
  const bool live = tok < a.T;
  const int64_t row_idx = ((int64_t)b * a.T + tok) * a.H + h;   // (b, tok, h)
  const E* vp = static_cast<const E*>(a.v);
  const E* dop = static_cast<const E*>(a.dout);
  const float* Hb = a.hs + tile * (int64_t)DK * a.Dv;
  const float* Db = a.dhs + tile * (int64_t)DK * a.Dv;

  float dPacc = 0.f, dAacc = 0.f;               // (t, i = j)
  float accB = 0.f, accG = 0.f, accW = 0.f;     // (t, column) partial sums
  float hdh = 0.f;
  float dQ[RB], dK[RB];
#pragma unroll
  for (int x = 0; x < RB; ++x) dQ[x] = dK[x] = 0.f;

  const int NV = a.Dv / 16;
  for (int jb = 0; jb < NV; ++jb) {
    const int col = 16 * jb;
    for (int x = tid; x < DK * 16; x += kBwdThreads) {
      const int rr = x >> 4, jj = x & 15;
      const float hv = Hb[(int64_t)rr * a.Dv + col + jj];
      const float dv = Db[(int64_t)rr * a.Dv + col + jj];
      sH[rr][jj] = hv;
      sD[rr][jj] = dv;
      hdh += hv * dv;
    }
    sV[t][j] = live ? ld1(vp + row_idx * a.Dv + col + j) : 0.f;
    sDO[t][j] = live ? ld1(dop + row_idx * a.Dv + col + j) : 0.f;
    __syncthreads();
    float KH = 0.f, QH = 0.f, KdH = 0.f;
#pragma unroll 8
    for (int rr = 0; rr < DK; ++rr) {
      KH += sK[t][rr] * sH[rr][j];
      QH += sQ[t][rr] * sH[rr][j];
      KdH += sK[t][rr] * sD[rr][j];
    }
    const float vres = sV[t][j] - sGam[t] * KH;
    sY[t][j] = sB[t] * vres;
    __syncthreads();
    float U = 0.f;
    for (int i = 0; i <= t; ++i) U += sTi[t][i] * sY[i][j];
    float dU = sEc[t] * KdH;
    for (int s = t; s < kT; ++s) dU += sP[s][t] * sDO[s][j];
    sU[t][j] = U;
    sDU[t][j] = dU;
    __syncthreads();
    float dY = 0.f;
    for (int s = t; s < kT; ++s) dY += sTi[s][t] * sDU[s][j];
    sDY[t][j] = dY;
    accB += dY * vres;
    accG += sGam[t] * QH * sDO[t][j] - sB[t] * sGam[t] * dY * KH;
    accW += sEc[t] * KdH * U;
    if (live) a.dv[row_idx * a.Dv + col + j] = sB[t] * dY;
    __syncthreads();
    // (t, i = j): dP = dO U^T, dA = -dY U^T
    {
      float p = 0.f, q = 0.f;
      for (int jj = 0; jj < 16; ++jj) {
        p += sDO[t][jj] * sU[j][jj];
        q += sDY[t][jj] * sU[j][jj];
      }
      dPacc += p;
      dAacc -= q;
    }
    // (t, rows j + 16x): dQ += gamma dO H^T; dK += -beta gamma dY H^T + ec U dH'^T
    {
      const float gq = sGam[t], gk = -sB[t] * sGam[t], ek = sEc[t];
#pragma unroll
      for (int x = 0; x < RB; ++x) {
        const int rr = j + 16 * x;
        float oh = 0.f, yh = 0.f, ud = 0.f;
        for (int jj = 0; jj < 16; ++jj) {
          oh += sDO[t][jj] * sH[rr][jj];
          yh += sDY[t][jj] * sH[rr][jj];
          ud += sU[t][jj] * sD[rr][jj];
        }
        dQ[x] += gq * oh;
        dK[x] += gk * yh + ek * ud;
      }
    }
    __syncthreads();
  }

  // intra-tile terms
  {
    const int i = j;
    const float e = i <= t ? __expf(sG[t] - sG[i]) : 0.f;
    const float dP = i <= t ? dPacc : 0.f;
    const float dA = i < t ? dAacc : 0.f;
    sPE[t][i] = dP * e;
    sM[t][i] = dA * sB[t] * e;
    sPP[t][i] = dP * sP[t][i];
    sAA[t][i] = dA * sB[t] * ekk;
    const float rb = sum16(accB), rg = sum16(accG), rw = sum16(accW), rak = sum16(dA * ekk);
    if (j == 0) {
      sRowB[t] = rb;
      sRowG[t] = rg;
      sRowW[t] = rw;
      sRowAK[t] = rak;
    }
    float hw = hdh;
    for (int m = 1; m < 64; m <<= 1) hw += __shfl_xor(hw, m, 64);
    if ((tid & 63) == 0) sHdH[tid >> 6] = hw;
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    const int rr = j + 16 * x;
    float q1 = 0.f, k1 = 0.f;
    for (int i = 0; i < kT; ++i) {
      q1 += sPE[t][i] * sK[i][rr];
      k1 += sPE[i][t] * sQ[i][rr] + sM[t][i] * sK[i][rr] + sM[i][t] * sK[i][rr];
    }
    dQ[x] += q1;
    dK[x] += k1;
  }
  if (live) {
    float* dqp = a.dq + row_idx * DK + j;
    float* dkp = a.dk + row_idx * DK + j;
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      dqp[16 * x] = dQ[x];
      dkp[16 * x] = dK[x];
    }
  }
  if (tid < kT) {
    // dg_u = sum_{t >= u} dG_t, with dG_t the gradient of the in-tile running
    // sum G_t.  The E-terms of P and A enter dG_t with + for the row and - for
    // the column, so their sum over t >= u keeps exactly the entries with row
    // >= u and column < u; the ec-terms keep the tokens before u; gamma_C
    // enters every u.  Summed in this form nothing large cancels.
    const int u = tid;
    float hd = 0.f;
    for (int w = 0; w < kBwdThreads / 64; ++w) hd += sHdH[w];
    float dg = gamC * hd;
    for (int i = 0; i < u; ++i) dg += sRowW[i];
    for (int t2 = u; t2 < kT; ++t2) {
      dg += sRowG[t2];
      for (int i = 0; i < u; ++i) dg += sPP[t2][i] + sAA[t2][i];
    }
    const int tk = c * kT + u;
    if (tk < a.T) {
      const int64_t idx = ((int64_t)b * a.T + tk) * a.H + h;
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
  const int64_t tiles = (int64_t)a.B * a.H * a.NT;
  const int64_t slices = (int64_t)a.B * a.H * (a.Dv / 16);
  hipLaunchKernelGGL((bwd_prep_kernel<E, DK>), dim3((unsigned)tiles), dim3(kBwdThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_hstates_kernel<E, DK>), dim3((unsigned)slices), dim3(kBwdThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dh_kernel<E, DK>), dim3((unsigned)slices), dim3(kBwdThreads), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_grad_kernel<E, DK>), dim3((unsigned)tiles), dim3(kBwdThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

long long chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv) {
  const long long nt = (T + kT - 1) / kT;
  const long long tiles = (long long)B * H * nt;
  return tiles * (BRec::FLOATS * 4LL + 2LL * Dk * Dv * 4LL);
}

hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const void* dout,
                            const float* gate, int gate_logit, float G, const float* beta,
                            const float* h0, const float* dhT, float* dq, float* dk, float* dv,
                            float* dgate, float* dbeta, float* dh0, int B, int T, int H, int Dk,
                            int Dv, int fp32, void* ws, hipStream_t st) {
  const int NT = (T + kT - 1) / kT;
  const int64_t tiles = (int64_t)B * H * NT;
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
  if (fp32) return Dk == 128 ? launch_bwd_t<float, 128>(a, st) : launch_bwd_t<float, 64>(a, st);
  return Dk == 128 ? launch_bwd_t<__bf16, 128>(a, st) : launch_bwd_t<__bf16, 64>(a, st);
}

}  // namespace la
