// la_bwd.h -- pieces shared by the two reverse-pass paths (chunk_bwd.hip, the
// float32-operand kernels, and chunk_bwd_bf16.hip, the bf16 matrix-core
// kernels): the per-tile record, the arguments, the maps from a grid index to
// (sequence, head, tile) and the per-tile preparation kernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "la_device.h"

namespace la {
namespace {

constexpr int kT = 16;          // tokens per tile
constexpr int kBwdThreads = 256;

// Workspace: per tile index (below: (b H + h) NT + c for a batch, h nslot +
// slot for packed sequences) a record, then the fp32 state at every tile
// start (hs) and the gradient of every tile's end state (dhs), each d_k x d_v
// per tile index, stored per 16-column slice in MFMA fragment order: element
// (row r, column 16 jb + n) of a tile's block sits at
// float ((jb * d_k / 16 + r / 16) * 64 + 16 ((r % 16) / 4) + n) * 4 + r % 4,
// so the serial kernels store whole 16-byte fragments.
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
  float* hs;    // [tile index][Dk x Dv] state at each tile start
  float* dhs;   // [tile index][Dk x Dv] gradient of each tile's end state
  int gate_logit;
  float G;
  int B, T, H, Dv, NT;
  const int* cu;   // packed sequences: nseq + 1 device offsets (B = nseq), or NULL
  int nslot;       // packed sequences: tile slots per head
  // bf16 path: states at the start of every second tile (hw, two per group)
  // and state gradients at every group end (dw), as packed bf16 hi | lo << 16
  // words per element; NG groups per sequence (batched) or nslotG group slots
  // per head (packed)
  unsigned* hw;
  unsigned* dw;
  int NG, nslotG;
  // bf16 path: the forward state after the last tile, float32 [B, H, Dk, Dv],
  // or NULL (the segmented reverse pass carries it to the next segment)
  float* hTo;
};

// One sequence of the call: T tokens from token tok0 of the token axis, NC
// tiles whose records, states and state gradients sit at tile indices rbase,
// rbase + 1, ...  Batched: sequence b of a.T tokens.  Packed (a.cu): tokens
// [cu[b], cu[b+1]) of one sequence of a.T tokens (offsets clamped to [0, a.T]
// and made non-decreasing); its tile c takes slot floor(cu[b] / 16) + b + c of
// the a.nslot = a.T / 16 + nseq + 1 per head (slots of different sequences do
// not overlap for non-decreasing offsets).
struct BSeq {
  int T, NC;
  int64_t tok0, rbase;
};
__device__ inline int bwd_begin(const BwdArgs& a, int s) { return min(max(a.cu[s], 0), a.T); }
__device__ inline BSeq bwd_seq(const BwdArgs& a, int b, int h) {
  BSeq q;
  if (a.cu) {
    const int tb = bwd_begin(a, b);
    q.T = min(max(a.cu[b + 1], tb), a.T) - tb;
    q.tok0 = tb;
    q.rbase = (int64_t)h * a.nslot + tb / 16 + b;
  } else {
    q.T = a.T;
    q.tok0 = (int64_t)b * a.T;
    q.rbase = ((int64_t)b * a.H + h) * a.NT;
  }
  q.NC = (q.T + 15) / 16;
  return q;
}
// A tile index of a grid over all tiles -> (sequence b, head h, tile c);
// false for a slot of a packed call that no tile uses.
__device__ inline bool bwd_tile(const BwdArgs& a, int64_t tile, int& b, int& h, int& c) {
  if (!a.cu) {
    c = (int)(tile % a.NT);
    const int64_t bh = tile / a.NT;
    h = (int)(bh % a.H);
    b = (int)(bh / a.H);
    return true;
  }
  h = (int)(tile / a.nslot);
  const int slot = (int)(tile - (int64_t)h * a.nslot);
  int lo = 0, hi = a.B - 1;                  // the last s with slot(s, 0) <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bwd_begin(a, mid) / 16 + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  b = lo;
  const BSeq q = bwd_seq(a, b, h);
  c = (int)(tile - q.rbase);
  return c >= 0 && c < q.NC;
}

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

// Rows of one tile of a [B, T, H, D] tensor into LDS (fp32, row pitch P),
// zeros past the end of the sequence.
template <typename E, int D, int P = D + 1>
__device__ inline void load_tile(float (*dst)[P], const E* src, const BSeq& sq, int c, int h,
                                 const BwdArgs& a) {
  constexpr int PER_ROW = D / 8;
  for (int x = threadIdx.x; x < kT * PER_ROW; x += kBwdThreads) {
    const int t = x / PER_ROW, c8 = (x % PER_ROW) * 8;
    const int tok = c * kT + t;
    float f[8];
    if (tok < sq.T) {
      Ld8<E>::run(src + ((sq.tok0 + tok) * a.H + h) * D + c8, f);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[t][c8 + i] = f[i];
  }
}

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
  int b, h, c;
  if (!bwd_tile(a, tile, b, h, c)) return;   // an unused slot: the whole block
  const BSeq sq = bwd_seq(a, b, h);
  load_tile<E, DK>(sK, static_cast<const E*>(a.k), sq, c, h, a);
  load_tile<E, DK>(sQ, static_cast<const E*>(a.q), sq, c, h, a);
  if (tid < kT) {
    const int tok = c * kT + tid;
    const int64_t idx = (sq.tok0 + tok) * a.H + h;
    sG[tid] = tok < sq.T ? gate_at(a, idx) : 0.f;
    sB[tid] = tok < sq.T ? a.beta[idx] : 0.f;
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

}  // namespace
}  // namespace la
