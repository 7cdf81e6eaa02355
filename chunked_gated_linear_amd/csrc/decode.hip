// decode.hip -- single-token recurrent update of the d_k x d_v state, in place.
//
// Constant-state recurrent inference: each (b, h) advances its state by one
// token ("Evaluating Next-Gen Sparse MoE and Long-Context LLMs", sec. 2 item 2
// and sec. 4).  With h = S^T and a = exp(g):
//     u   = beta * (v - a * h^T k)                      (d_v)
//     h'  = a * h + k u^T                               (one pass over h)
//     o   = h'^T q = a * h^T q + (k . q) u
// so h is read once and written once; both column reductions (h^T k, h^T q)
// come from the same register-resident copy.
//
// Roofline: 2 * Dk * Dv * 4 bytes of state traffic per head and step dominate
// (about 9 * Dk * Dv flops against 8 * Dk * Dv bytes): HBM-bound.
//
// Layout: a persistent grid of 1024-thread workgroups, four per compute unit,
// walks the (b, h) list in steps of the grid size, so that the heads in flight
// at any time are neighbours in memory (at B = 256, H = 32, d = 128 this ran
// at 6.1 TB/s against 5.7 with 512-thread workgroups, eight per unit).  Thread (rg, c4) holds columns 4*c4 .. 4*c4+3 of rows
// rg, rg + RG, rg + 2*RG, ... as float4, so every row of the state is read and
// written as consecutive 16-byte pieces.  The state is streamed once per step
// (it does not fit the last-level cache), so its loads and stores are marked
// non-temporal.
#include <atomic>

#include "la_device.h"
#include "la_launch.h"

namespace la {

int device_cus() {
  static std::atomic<int> cache[64];   // 0 = not queried yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  const bool slot = dev >= 0 && dev < 64;
  if (slot) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  if (slot) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

constexpr int kDecodeThreads = 1024;
constexpr int kDecodeBlocksPerCU = 4;

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ gate, int gate_logit, float G,
    const float* __restrict__ beta, float* __restrict__ S, E* __restrict__ o, int BH) {
  constexpr int NC4 = DV / 4;                  // float4 columns per row
  constexpr int RG = kDecodeThreads / NC4;     // row groups
  constexpr int RPT = DK / RG;                 // rows per thread
  static_assert(RG * NC4 == kDecodeThreads && RPT * RG == DK, "decode tiling");
  static_assert(DK <= kDecodeThreads && DV <= kDecodeThreads, "one thread per element of k, q, v");

  __shared__ float sk[DK], sq[DK];
  __shared__ f32x4 pa[RG][NC4], pb[RG][NC4];
  __shared__ float su[DV];
  __shared__ float skq;

  const int tid = threadIdx.x;
  const int c4 = tid % NC4, rg = tid / NC4;

  for (int64_t bh = blockIdx.x; bh < BH; bh += gridDim.x) {
    const float gx = gate[bh];
    const float g = gate_logit ? bounded_gate(gx, G) : gx;
    const float a = __expf(g);
    const float bt = beta[bh];

    if (tid < DK) {
      sk[tid] = Elt<E>::to_f(k[bh * DK + tid]);
      sq[tid] = Elt<E>::to_f(q[bh * DK + tid]);
    }
    f32x4* Sh = reinterpret_cast<f32x4*>(S + bh * DK * DV);
    f32x4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = __builtin_nontemporal_load(Sh + (rg + RG * i) * NC4 + c4);
    __syncthreads();

    f32x4 pk = zero4(), pq = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      pk += sk[rg + RG * i] * s[i];
      pq += sq[rg + RG * i] * s[i];
    }
    pa[rg][c4] = pk;
    pb[rg][c4] = pq;
    if (tid < 64) {  // k . q, one wave, fixed order
      float p = 0.f;
      for (int d = tid; d < DK; d += 64) p += sk[d] * sq[d];
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
      const float u = bt * (Elt<E>::to_f(v[bh * DV + tid]) - a * hk);
      su[tid] = u;
      o[bh * DV + tid] = Elt<E>::from_f(a * hq + skq * u);
    }
    __syncthreads();

    const f32x4 u4 = reinterpret_cast<const f32x4*>(su)[c4];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      __builtin_nontemporal_store(a * s[i] + sk[rg + RG * i] * u4, Sh + (rg + RG * i) * NC4 + c4);
    __syncthreads();   // the shared buffers are reused by the next (b, h)
  }
}

template <typename E, int DK, int DV>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v,
                                  const float* gate, int gate_logit, float G,
                                  const float* beta, float* S, void* o, int BH,
                                  hipStream_t st) {
  const int cap = kDecodeBlocksPerCU * device_cus();
  const int grid = BH < cap ? BH : cap;
  hipLaunchKernelGGL((decode_kernel<E, DK, DV>), dim3(grid), dim3(kDecodeThreads), 0, st,
                     (const E*)q, (const E*)k, (const E*)v, gate, gate_logit, G,
                     beta, S, (E*)o, BH);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* gate, int gate_logit, float G,
                         const float* beta, float* S, void* o, int BH, int Dk,
                         int Dv, int fp32, hipStream_t st) {
#define LA_DEC(E, DK, DV) \
  if (Dk == DK && Dv == DV) return launch_decode_t<E, DK, DV>(q, k, v, gate, gate_logit, G, beta, S, o, BH, st);
  if (fp32) {
    LA_DEC(float, 64, 64) LA_DEC(float, 64, 128) LA_DEC(float, 128, 64) LA_DEC(float, 128, 128)
  } else {
    LA_DEC(__bf16, 64, 64) LA_DEC(__bf16, 64, 128) LA_DEC(__bf16, 128, 64) LA_DEC(__bf16, 128, 128)
  }
#undef LA_DEC
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Bounded log-decay on its own, g = -G * sigmoid(x) ("Deep Dive: The Next
// Generation of Ultra-Long Context Sparse MoE LLMs", sec. 3.3).  Elementwise,
// HBM-bound; grid-stride loop.
__global__ __launch_bounds__(256) void gate_kernel(const float* x, float G, float* g,
                                                   long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    g[i] = bounded_gate(x[i], G);
}

hipError_t launch_gate(const float* x, float G, float* g, long long n, hipStream_t st) {
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, G, g, n);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_kernel(float* p, long long n, float val) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    p[i] = val;
}

__global__ __launch_bounds__(256) void copy_kernel(const float* s, float* d, long long n) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    d[i] = s[i];
}

hipError_t launch_state_init(const float* h0, float* hT, long long n, hipStream_t st) {
  long long blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (h0)
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st, h0, hT, n);
  else
    hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, st, hT, n, 0.0f);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Debug range check of a forward pass's inputs: the bounded log-decay lies in
// [-G, 0] ("Deep Dive: The Next Generation of Ultra-Long Context Sparse MoE
// LLMs", sec. 3.3), beta in [0, 1], everything finite.  Grid-stride over each
// array; per-wave OR of the flags, then one atomic OR per wave that found
// anything (the result does not depend on the order).
__global__ void clear_flag_kernel(unsigned* flags) { flags[0] = 0u; }

template <typename E>
__device__ inline bool fin(E x) { return __builtin_isfinite((float)x); }

template <typename E>
__global__ __launch_bounds__(256) void range_kernel(const E* q, const E* k, long long nqk,
                                                    const E* v, long long nv, const float* gate,
                                                    long long ngate, int gate_logit, float G,
                                                    const float* beta, long long nbeta,
                                                    const float* h0, long long nh0,
                                                    unsigned* flags) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long i0 = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned f = 0;
  for (long long i = i0; i < nqk; i += stride)
    if (!fin(q[i]) || !fin(k[i])) f |= 1u;
  for (long long i = i0; i < nv; i += stride)
    if (!fin(v[i])) f |= 1u;
  for (long long i = i0; i < ngate; i += stride) {
    const float x = gate[i];
    if (gate_logit ? x != x : !(x >= -G && x <= 0.f)) f |= 2u;
  }
  for (long long i = i0; i < nbeta; i += stride) {
    const float x = beta[i];
    if (!(x >= 0.f && x <= 1.f)) f |= 4u;
  }
  for (long long i = i0; i < nh0; i += stride)
    if (!__builtin_isfinite(h0[i])) f |= 8u;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) f |= (unsigned)__shfl_xor((int)f, d);
  if ((threadIdx.x & 63) == 0 && f) atomicOr(flags, f);
}

hipError_t launch_range_check(const void* q, const void* k, const void* v, const float* gate,
                              int gate_logit, float G, const float* beta, const float* h0,
                              long long nqk, long long nv, long long ngate, long long nbeta,
                              long long nh0, int fp32, unsigned* flags, hipStream_t st) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, st, flags);
  const long long n = nqk > ngate ? nqk : ngate;
  long long blocks = (n + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  if (fp32)
    hipLaunchKernelGGL(range_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const float*)q, (const float*)k, nqk, (const float*)v, nv, gate, ngate,
                       gate_logit, G, beta, nbeta, h0, h0 ? nh0 : 0, flags);
  else
    hipLaunchKernelGGL(range_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, st,
                       (const __bf16*)q, (const __bf16*)k, nqk, (const __bf16*)v, nv, gate, ngate,
                       gate_logit, G, beta, nbeta, h0, h0 ? nh0 : 0, flags);
  return hipGetLastError();
}

}  // namespace la
