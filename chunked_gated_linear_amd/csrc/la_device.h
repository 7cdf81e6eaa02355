// la_device.h -- device-side building blocks for the gfx950 kernels:
// element types, MFMA fragment types and wrappers, conversions.
//
// Fragment conventions (16x16 output tiles, wave64, lane l = 16*grp + n):
//   accumulator  : lane l holds D[4*grp + i][n], i = 0..3           (f32x4)
//   16-deep A/B  : lane l holds M[n][kappa16(grp, j)], j = 0..3     (frag16)
//   32-deep A/B  : lane l holds M[n][kappa32(grp, j)], j = 0..7     (frag32)
// where for A the row is the output row and for B the row is the output
// column (B is passed "transposed", as its columns).  The hardware contracts
// A's (grp, j) with B's (grp, j); which contraction index a (grp, j) pair
// stands for is our choice, made identically on both sides:
//   kappa16(grp, j) = 4*grp + j
//   kappa32(grp, j) = 16*(j >> 2) + 4*grp + (j & 3)
// With these, an accumulator tile is already a 16-deep B fragment, and the
// accumulator tiles 2s and 2s+1 of a 16-row-tiled matrix together are the
// 32-deep B fragment for contraction block s.  No lane shuffles are needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Element-type traits: storage type, 16- and 32-deep fragments, MFMA wrappers.
template <typename E> struct Elt;

template <> struct Elt<__bf16> {
  typedef __bf16 T;
  struct F16 { bf16x4 v; };
  struct F32 { bf16x8 v; };
  static constexpr int kBytes = 2;
  __device__ static inline f32x4 mma16(const F16& a, const F16& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
        __builtin_bit_cast(s16x4, a.v), __builtin_bit_cast(s16x4, b.v), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mma32(const F32& a, const F32& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
  }
  __device__ static inline F16 from_acc(f32x4 x) {
    F16 r;
    r.v = bf16x4{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    return r;
  }
  // 32-deep fragment from two accumulator tiles (lo = tile 2s, hi = tile 2s+1).
  __device__ static inline F32 from_acc2(f32x4 lo, f32x4 hi) {
    F32 r;
    r.v = bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                 (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
    return r;
  }
  // The 16-deep half h (0 or 1) of a 32-deep fragment.
  __device__ static inline F16 half(const F32& a, int h) {
    F16 r;
    r.v = h ? bf16x4{a.v[4], a.v[5], a.v[6], a.v[7]} : bf16x4{a.v[0], a.v[1], a.v[2], a.v[3]};
    return r;
  }
  __device__ static inline float to_f(T x) { return (float)x; }
  __device__ static inline T from_f(float x) { return (T)x; }
};

template <> struct Elt<float> {
  typedef float T;
  struct F16 { f32x4 v; };
  struct F32 { f32x4 lo, hi; };
  static constexpr int kBytes = 4;
  // fp32 MFMA 16x16x4: lane l holds A[n][grp] (resp. B), one value; four (resp.
  // eight) of them make up a 16- (32-) deep product.  Register j of lane
  // (n, grp) is contracted with register j of the partner lane, so the kappa
  // conventions above hold unchanged.
  __device__ static inline f32x4 mma16(const F16& a, const F16& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[0], b.v[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[1], b.v[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[2], b.v[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[3], b.v[3], c, 0, 0, 0);
    return c;
  }
  __device__ static inline f32x4 mma32(const F32& a, const F32& b, f32x4 c) {
    F16 alo{a.lo}, ahi{a.hi}, blo{b.lo}, bhi{b.hi};
    c = mma16(alo, blo, c);
    return mma16(ahi, bhi, c);
  }
  __device__ static inline F16 from_acc(f32x4 x) { return F16{x}; }
  __device__ static inline F32 from_acc2(f32x4 lo, f32x4 hi) { return F32{lo, hi}; }
  __device__ static inline F16 half(const F32& a, int h) { return F16{h ? a.hi : a.lo}; }
  __device__ static inline float to_f(T x) { return x; }
  __device__ static inline T from_f(float x) { return x; }
};

__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Bounded log-decay g = -G * sigmoid(x) with the hardware exponential and
// reciprocal (about 1 ulp each).  Saturates cleanly: for very negative x the
// exponential is +inf, its reciprocal 0 and g = -0; for very positive x it is
// 0 and g = -G.
__device__ inline float bounded_gate(float x, float G) {
  return -G * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// Logistic function 1 / (1 + exp(-x)) with the same hardware exponential and
// reciprocal as bounded_gate.
__device__ inline float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Lane-group (16 lanes) inclusive prefix sum; every 16-lane group scans its
// own values independently.
__device__ inline float scan16(float x, int n) {
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
    float y = __shfl_up(x, d, 16);
    if (n >= d) x += y;
  }
  return x;
}

}  // namespace la
