// la_bwd_bf16.h -- pieces shared by the bf16 reverse-pass kernels
// (chunk_bwd_bf16.hip: tile records and gradients; chunk_bwd_bf16_states.hip:
// the two serial chains): checkpoint spacing, the bf16 hi / lo split and
// MFMA helpers, the LDS row and slab layouts, and the launch of the chains.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "la_bwd.h"
#include "la_device.h"

namespace la {
namespace {

constexpr int kGS = 4;          // tiles per checkpoint group
constexpr int kHS = 2;          // tiles per stored start state (kGS / kHS of them per group)
constexpr int kHPG = kGS / kHS;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;

// ------------------------------------------------------------- helpers
__device__ inline bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ inline bf16x4 first4(bf16x8 a) { return bf16x4{a[0], a[1], a[2], a[3]}; }
__device__ inline bf16x4 second4(bf16x8 a) { return bf16x4{a[4], a[5], a[6], a[7]}; }
__device__ inline f32x4 mma32b(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// [A_hi | A_lo] . [B_lo ; 0] = A_hi B_lo: the third term of a split-by-split
// 16-deep product, as a 32-deep MFMA with a zero half.  Every product here is
// a 16x16x32 MFMA: a 16x16x16 one reading, as its accumulator, the result of a
// 16x16x32 MFMA issued just before came out wrong in accumulator registers 0
// and 1 in this build (the instructions between them did not cover the
// dependency).
__device__ inline f32x4 mma32b_lo(bf16x8 a, bf16x4 blo, f32x4 c) {
  return mma32b(a, cat8(blo, bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f}), c);
}
__device__ inline f32x4 to_f4(bf16x4 x) {
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// A float32 fragment as bf16 hi + lo parts: hi is x rounded to bf16, lo is
// the remainder x - hi (exact in float32) rounded to bf16, so |x - hi - lo|
// <= 2^-17 |x|.  Three instructions per element: each pair is converted to a
// packed bf16 word once, its halves are widened back by a shift and a mask
// for the subtraction, and the remainders are converted as a pair.
struct Sp4 {
  bf16x4 h, l;
};
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ inline Sp4 split4(f32x4 x) {
  const unsigned p01 = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{x[0], x[1]}), bf16x2));
  const unsigned p23 = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2{x[2], x[3]}), bf16x2));
  const f32x2 r01 = f32x2{x[0] - __uint_as_float(p01 << 16), x[1] - __uint_as_float(p01 & 0xffff0000u)};
  const f32x2 r23 = f32x2{x[2] - __uint_as_float(p23 << 16), x[3] - __uint_as_float(p23 & 0xffff0000u)};
  Sp4 s;
  s.h = __builtin_bit_cast(bf16x4, uint2{p01, p23});
  s.l = __builtin_bit_cast(bf16x4, uint2{__builtin_bit_cast(unsigned, __builtin_convertvector(r01, bf16x2)),
                                         __builtin_bit_cast(unsigned, __builtin_convertvector(r23, bf16x2))});
  return s;
}

// Packed checkpoint words: element = bf16 hi in bits 0..15, bf16 lo in 16..31.
__device__ inline uint4 pack_words(bf16x4 h, bf16x4 l) {
  const s16x4 hs = __builtin_bit_cast(s16x4, h), ls = __builtin_bit_cast(s16x4, l);
  uint4 w;
  w.x = (unsigned)(unsigned short)hs[0] | ((unsigned)(unsigned short)ls[0] << 16);
  w.y = (unsigned)(unsigned short)hs[1] | ((unsigned)(unsigned short)ls[1] << 16);
  w.z = (unsigned)(unsigned short)hs[2] | ((unsigned)(unsigned short)ls[2] << 16);
  w.w = (unsigned)(unsigned short)hs[3] | ((unsigned)(unsigned short)ls[3] << 16);
  return w;
}
__device__ inline float word_f(unsigned w) {
  return __uint_as_float(w << 16) + __uint_as_float(w & 0xffff0000u);
}
__device__ inline f32x4 words_f4(uint4 w) {
  return f32x4{word_f(w.x), word_f(w.y), word_f(w.z), word_f(w.w)};
}

// Packed words -> the bf16 hi and lo parts of four elements.
__device__ inline void words_split(uint4 w, bf16x4& h, bf16x4& l) {
  const unsigned h01 = (w.x & 0xffffu) | (w.y << 16), h23 = (w.z & 0xffffu) | (w.w << 16);
  const unsigned l01 = (w.x >> 16) | (w.y & 0xffff0000u), l23 = (w.z >> 16) | (w.w & 0xffff0000u);
  h = __builtin_bit_cast(bf16x4, uint2{h01, h23});
  l = __builtin_bit_cast(bf16x4, uint2{l01, l23});
}
// The split fragments of a state stored as packed words (tile t at w[t]).
template <int NS>
__device__ inline void words_state(const uint4* w, int stride, bf16x8* sh, bf16x8* sl) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    bf16x4 ah, al, bh, bl;
    words_split(w[(2 * s) * stride], ah, al);
    words_split(w[(2 * s + 1) * stride], bh, bl);
    sh[s] = cat8(ah, bh);
    sl[s] = cat8(al, bl);
  }
}

// The split fragments of a d_k x 16 state held as NT float32 accumulator
// tiles: 32-deep B fragments of contraction block s (tiles 2s and 2s + 1).
template <int NS>
__device__ inline void split_state(const f32x4* acc, bf16x8* sh, bf16x8* sl) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const Sp4 a = split4(acc[2 * s]), b = split4(acc[2 * s + 1]);
    sh[s] = cat8(a.h, b.h);
    sl[s] = cat8(a.l, b.l);
  }
}

// 16 x 16 bf16 tile, accumulator layout (lane (n, grp) holds X[4 grp + i][n])
// -> row layout (lane (n, grp) holds X[n][4 grp + j]) through 512 bytes of
// this wave's LDS: a lane-order write, then a transposing read in which lane
// (n, grp) points at the 8 bytes written by lane (4 grp + n / 4, n % 4).
__device__ inline void tr_put(char* buf, int lane, bf16x4 x) {
  *reinterpret_cast<bf16x4*>(buf + 8 * lane) = x;
}
__device__ inline bf16x4 tr_get(char* buf, int n, int grp) {
  const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(buf + 8 * (16 * (n & 3) + 4 * grp + (n >> 2))));
  return __builtin_bit_cast(bf16x4, r);
}
// Sum over each 16-lane row of the wave by an inclusive scan (DPP row_shr 1,
// 2, 4, 8, zeros shifted in): lane 15 of the row ends with the row's total.
__device__ inline float rowsum16(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  return x;
}
__device__ inline void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Token rows of one tile of k or q in LDS, bf16, row pitch 2 DK + 16 bytes
// (the pad spreads the rows of a fragment read over the banks).
//   A fragment of block s (32-deep over d_k): lane (n, grp) holds
//     K[n][32 s + kappa32(grp, j)]: two 8-byte reads of row n;
//   transposed A fragment of 16-row block t (16-deep over tokens): lane
//     (n, grp) holds K[4 grp + j][16 t + n]: one transposing read in which
//     lane (n, grp) points at row 4 grp + n / 4, columns 16 t + 4 (n % 4).
template <int DK>
struct Rows {
  static constexpr int PITCH = 2 * DK + 16;
  static constexpr int BYTES = 16 * PITCH;
  __device__ static inline bf16x8 afrag(const char* rows, int s, int n, int grp) {
    const char* p = rows + n * PITCH + 2 * (32 * s + 4 * grp);
    return cat8(*reinterpret_cast<const bf16x4*>(p), *reinterpret_cast<const bf16x4*>(p + 32));
  }
  __device__ static inline bf16x4 tfrag(const char* rows, int t, int n, int grp) {
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(rows + (4 * grp + (n >> 2)) * PITCH + 32 * t + 8 * (n & 3)));
    return __builtin_bit_cast(bf16x4, r);
  }
};

// 16 token rows of SPW 16-column slices of v or dout (bf16) in LDS, row pitch
// 32 SPW + 16 bytes: staged as 16-byte pieces (lane l's piece x is piece
// 64 x + l in row-major order, PR to a row), read back per slice w in the
// accumulator layout (lane (n, grp) holds X[4 grp + j][16 w + n]) by one
// transposing read, as Rows::tfrag.
template <int SPW>
struct Slab {
  static constexpr int PITCH = 32 * SPW + 16;
  static constexpr int BYTES = 16 * PITCH;
  static constexpr int PR = 2 * SPW;
  static constexpr int NPC = (16 * PR + 63) / 64;
  __device__ static inline bf16x4 get(const char* slab, int w, int n, int grp) {
    const s16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(slab + (4 * grp + (n >> 2)) * PITCH + 32 * w + 8 * (n & 3)));
    return __builtin_bit_cast(bf16x4, r);
  }
  // this lane's pieces of the tile whose token 0 is at `base` (column 0 of the
  // slices), rows past `last` read row `last`
  __device__ static inline void load(uint4* out, const __bf16* base, int stride, int last, int lane) {
#pragma unroll
    for (int x = 0; x < NPC; ++x) {
      const int pc = min(64 * x + lane, 16 * PR - 1);
      out[x] = *reinterpret_cast<const uint4*>(base + min(pc / PR, last) * stride + 8 * (pc % PR));
    }
  }
  // stage them; rows at or past `nrows` as zeros
  template <bool CHK>
  __device__ static inline void stage(char* slab, const uint4* in, int nrows, int lane) {
#pragma unroll
    for (int x = 0; x < NPC; ++x) {
      const int pc = 64 * x + lane;
      if (16 * PR % 64 == 0 || pc < 16 * PR) {
        const int row = pc / PR;
        *reinterpret_cast<uint4*>(slab + row * PITCH + 16 * (pc % PR)) =
            (!CHK || row < nrows) ? in[x] : uint4{0u, 0u, 0u, 0u};
      }
    }
  }
};

// Index of group 0 of sequence b, head h in the checkpoint arrays.
__device__ inline int64_t grp_base(const BwdArgs& a, int b, int h) {
  if (a.cu) return (int64_t)h * a.nslotG + bwd_begin(a, b) / (16 * kGS) + b;
  return ((int64_t)b * a.H + h) * a.NG;
}

// A group slot of the gradient grid -> (sequence b, head h, group g); false
// for a slot no group uses.
__device__ inline bool bwd2_group(const BwdArgs& a, int64_t blk, int& b, int& h, int& g) {
  if (!a.cu) {
    g = (int)(blk % a.NG);
    const int64_t bh = blk / a.NG;
    h = (int)(bh % a.H);
    b = (int)(bh / a.H);
    return 16 * kGS * g < a.T;
  }
  h = (int)(blk / a.nslotG);
  const int slot = (int)(blk - (int64_t)h * a.nslotG);
  int lo = 0, hi = a.B - 1;                  // the last s whose group 0 sits at or before slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bwd_begin(a, mid) / (16 * kGS) + mid <= slot) lo = mid;
    else hi = mid - 1;
  }
  b = lo;
  const BSeq sq = bwd_seq(a, b, h);
  g = slot - (bwd_begin(a, b) / (16 * kGS) + b);
  return g >= 0 && kGS * g < sq.NC;
}

// Per-tile operator fragments built from the record's row-major float32 16 x
// 16 matrices: element (t, i) of M as a split A fragment [M_hi | M_lo] (lane
// (n = t, grp = i / 4), register i % 4), or of M^T (lane (n = i, grp = t / 4),
// register t % 4).  `frag` is 64 lanes x 16 bytes.
__device__ inline void put_op(char* frag, int t, int i, float x, bool transposed) {
  const int n = transposed ? i : t, c = transposed ? t : i;
  char* p = frag + 16 * (16 * (c >> 2) + n) + 2 * (c & 3);
  const __bf16 hb = (__bf16)x;
  *reinterpret_cast<__bf16*>(p) = hb;
  *reinterpret_cast<__bf16*>(p + 8) = (__bf16)(x - (float)hb);
}

__device__ inline uint4 zero_if(bool ok, uint4 x) { return ok ? x : uint4{0u, 0u, 0u, 0u}; }
__device__ inline bf16x8 u4_bf8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

static_assert(std::is_trivially_copyable<BwdArgs>::value, "BwdArgs crosses files as bytes");

}  // namespace

// The launch of the forward-state and state-gradient chains
// (chunk_bwd_bf16_states.hip): `args` is the caller's BwdArgs (args_bytes =
// its size, checked), Dk = d_k, grid = nblk or 2 nblk workgroups of spw
// slices each.  Returns hipErrorInvalidValue for a size, d_k or slice count it
// does not take, else the launch status.
hipError_t launch_bwd_bf16_states(const void* args, size_t args_bytes, int Dk, int spw, unsigned grid,
                                  int nblk, hipStream_t st);

}  // namespace la
