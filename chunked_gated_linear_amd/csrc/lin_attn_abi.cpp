// lin_attn_abi.cpp -- the C ABI declared in include/lin_attn.h: host-side
// argument checks, then one launch on the caller's stream.  Nothing here
// touches the device before every check has passed.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <string>
#include <utility>

#include "la_launch.h"
#include "lin_attn.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return LA_OK;
}

struct Span {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const char* name, const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{name, a, a + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(const Span& a, const Span& b) {
  if (!a.lo || !b.lo || a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1u)) == 0; }

int check_gate_scalars(int gate_mode, float G) {
  if (gate_mode != LA_GATE_LOG && gate_mode != LA_GATE_BOUNDED_LOGIT)
    return fail(LA_EINVAL, "gate_mode must be LA_GATE_LOG (0) or LA_GATE_BOUNDED_LOGIT (1), got %d",
                gate_mode);
  if (!std::isfinite(G) || G < 0.f || G > 16.f)
    return fail(LA_ERANGE, "G must be finite and in [0, 16], got %g", (double)G);
  return LA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Size checks shared by lin_attn_chunk_fwd and its workspace query.
int check_chunk_sizes(int B, int T, int H, int Dk, int Dv, int dtype) {
  if (B < 0 || T < 0 || H < 0)
    return fail(LA_EINVAL, "sizes must be >= 0 (B=%d T=%d H=%d)", B, T, H);
  if (dtype != LA_BF16 && dtype != LA_FP32)
    return fail(LA_EINVAL, "dtype must be LA_BF16 (0) or LA_FP32 (1), got %d", dtype);
  if (Dk != 64 && Dk != 128)
    return fail(LA_EUNSUPPORTED, "Dk must be 64 or 128, got %d", Dk);
  if (Dv < 16 || Dv > 256 || Dv % 16 != 0)
    return fail(LA_EUNSUPPORTED, "Dv must be a multiple of 16 in [16, 256], got %d", Dv);
  const int64_t ntok = (int64_t)B * T * H;
  if ((int64_t)B * H * (Dv / 16) > INT32_MAX || ntok > (INT64_C(1) << 40))
    return fail(LA_EINVAL, "problem too large (B*H*Dv/16 = %lld)",
                (long long)((int64_t)B * H * (Dv / 16)));
  if ((int64_t)T * H * (Dk > Dv ? Dk : Dv) > INT32_MAX || (int64_t)B * T > INT32_MAX)
    return fail(LA_EINVAL, "problem too large (T*H*max(Dk,Dv) or B*T exceeds 2^31)");
  return LA_OK;
}

// Size checks shared by lin_attn_chunk_fwd_varlen and its workspace query.
int check_varlen_sizes(int T, int nseq, int H, int Dk, int Dv, int dtype) {
  if (nseq < 0) return fail(LA_EINVAL, "nseq must be >= 0, got %d", nseq);
  if (int rc = check_chunk_sizes(nseq > 0 ? 1 : 0, T, H, Dk, Dv, dtype)) return rc;
  if ((int64_t)nseq * H * (Dv / 16) > INT32_MAX || (int64_t)T / 32 + nseq + 1 > INT32_MAX / 2)
    return fail(LA_EINVAL, "problem too large (nseq = %d)", nseq);
  return LA_OK;
}

// The per-head scale and shift of the gate logit (either may be NULL):
// 4-byte aligned device arrays of H floats, disjoint from every output.
int check_gate_affine(const float* gsc, const float* gbi, int H, const void* o, int64_t o_bytes,
                      const float* hT, int64_t hT_bytes, const void* ws, int64_t ws_bytes) {
  const struct { const char* nm; const float* p; } arr[] = {{"gate_scale", gsc},
                                                           {"gate_bias", gbi}};
  for (const auto& a : arr) {
    if (!a.p) continue;
    if (!aligned(a.p, 4u)) return fail(LA_EINVAL, "%s must be 4-byte aligned", a.nm);
    const Span sa = span(a.nm, a.p, (int64_t)H * 4);
    const Span outs[] = {span("o", o, o_bytes), span("hT", hT, hT_bytes),
                         span("workspace", ws, ws_bytes)};
    for (const Span& out : outs)
      if (overlap(out, sa)) return fail(LA_EINVAL, "%s overlaps %s", out.name, a.nm);
  }
  return LA_OK;
}

long long chunk_workspace(int B, int T, int H, int Dk, int Dv, int dtype) {
  return dtype == LA_BF16 ? la::chunk_pair_workspace_bytes(B, T, H, Dk, Dv) : 0;
}

long long channel_workspace(int B, int T, int H, int Dk, int Dv, int dtype) {
  return T > 0 ? la::chunk_channel_workspace_bytes(B, T, H, Dk, Dv, dtype == LA_FP32) : 0;
}

}  // namespace

extern "C" {

const char* lin_attn_last_error(void) { return g_err.c_str(); }

int lin_attn_check_inputs(const void* q, const void* k, const void* v, const float* gate,
                          int gate_mode, float G, const float* beta, const float* h0,
                          long long ntok, int nstate, int H, int Dk, int Dv, int channel,
                          int dtype, unsigned* flags, void* stream) {
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  if (ntok < 0 || nstate < 0 || H < 0 || Dk < 1 || Dv < 1 || Dk > 4096 || Dv > 4096)
    return fail(LA_EINVAL, "bad sizes (ntok=%lld nstate=%d H=%d Dk=%d Dv=%d)", ntok, nstate, H,
                Dk, Dv);
  if (dtype != LA_BF16 && dtype != LA_FP32)
    return fail(LA_EINVAL, "dtype must be LA_BF16 (0) or LA_FP32 (1), got %d", dtype);
  if (!flags || !aligned(flags, 4u)) return fail(LA_EINVAL, "flags must be a 4-byte aligned pointer");
  const int64_t nqk = (int64_t)ntok * H * Dk, nv = (int64_t)ntok * H * Dv;
  const int64_t ngate = (int64_t)ntok * H * (channel ? Dk : 1), nbeta = (int64_t)ntok * H;
  const int64_t nh0 = (int64_t)nstate * H * Dk * Dv;
  if (nqk > 0) {
    const struct { const char* nm; const void* p; } req[] = {
        {"q", q}, {"k", k}, {"v", v}, {"gate", gate}, {"beta", beta}};
    for (const auto& r : req) {
      if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
      if (!aligned(r.p, dtype == LA_BF16 ? 2u : 4u)) return fail(LA_EINVAL, "%s misaligned", r.nm);
    }
  }
  if (h0 && !aligned(h0, 4u)) return fail(LA_EINVAL, "h0 must be 4-byte aligned");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (int rc = hip_status(la::launch_range_check(q, k, v, gate, gate_mode == LA_GATE_BOUNDED_LOGIT,
                                                 G, beta, h0, nqk, nv, ngate, nbeta, nh0,
                                                 dtype == LA_FP32, flags, st),
                          "range check launch"))
    return rc;
  unsigned f = 0;
  if (int rc = hip_status(hipStreamSynchronize(st), "range check")) return rc;
  if (int rc = hip_status(hipMemcpy(&f, flags, sizeof f, hipMemcpyDeviceToHost), "range check copy"))
    return rc;
  if (!f) return ok();
  std::string m = "inputs out of range:";
  if (f & 1u) m += " non-finite q, k or v;";
  if (f & 2u) m += gate_mode == LA_GATE_LOG ? " gate outside [-G, 0] or non-finite;" : " NaN gate logit;";
  if (f & 4u) m += " beta outside [0, 1];";
  if (f & 8u) m += " non-finite h0;";
  return fail(LA_ERANGE, "%s", m.c_str());
}

int lin_attn_version(void) { return 200; }

long long lin_attn_chunk_fwd_workspace_size(int B, int T, int H, int Dk, int Dv, int dtype) {
  if (check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return -1;
  ok();
  return chunk_workspace(B, T, H, Dk, Dv, dtype);
}

}  // extern "C"

namespace {

// lin_attn_chunk_fwd (raw = 0) and lin_attn_chunk_fwd_raw (raw = 1).
int chunk_fwd(const void* q, const void* k, const void* v, const float* gate, int gate_mode,
              float G, const float* beta, const float* h0, void* o, float* hT, int B, int T,
              int H, int Dk, int Dv, int dtype, void* workspace, long long workspace_bytes,
              void* stream, int raw, int channel = 0, const float* gsc = nullptr,
              const float* gbi = nullptr) {
  if (int rc = check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return rc;
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  // per-channel gate: the in-tile operands reach exp(+-8 G); G <= 10 keeps
  // them at most exp(80), inside the float range
  if (channel && G > 10.f)
    return fail(LA_ERANGE, "G must be in [0, 10] for a per-channel gate, got %g", (double)G);
  const int64_t es = dtype == LA_BF16 ? 2 : 4;
  const int64_t ntok = (int64_t)B * T * H;
  const int64_t nst = (int64_t)B * H * Dk * Dv;
  if (B == 0 || H == 0) return ok();
  const unsigned ea = dtype == LA_BF16 ? 2u : 4u;
  const long long wsz = T <= 0 ? 0
                        : channel ? channel_workspace(B, T, H, Dk, Dv, dtype)
                                  : chunk_workspace(B, T, H, Dk, Dv, dtype);
  const int64_t ngate = channel ? ntok * Dk : ntok;   // gate elements
  if (T > 0) {
    // q, k and v are read as 16-byte vectors, bf16 o written as 8-byte vectors;
    // gate and beta element-wise
    const struct { const char* nm; const void* p; unsigned a; } req[] = {
        {"q", q, 16u}, {"k", k, 16u}, {"v", v, 16u}, {"gate", gate, channel ? 16u : 4u},
        {"beta", beta, 4u},
        {"o", o, dtype == LA_BF16 ? 8u : ea}};
    for (const auto& r : req) {
      if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
      if (!aligned(r.p, r.a)) return fail(LA_EINVAL, "%s must be %u-byte aligned", r.nm, r.a);
    }
  }
  if (h0 && !aligned(h0, 4u)) return fail(LA_EINVAL, "h0 must be 4-byte aligned");
  if (hT && !aligned(hT, 4u)) return fail(LA_EINVAL, "hT must be 4-byte aligned");
  if (wsz > 0) {
    if (!workspace) return fail(LA_EINVAL, "workspace must not be NULL (%lld bytes needed)", wsz);
    if (!aligned(workspace, 256u)) return fail(LA_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < wsz)
      return fail(LA_EINVAL, "workspace too small: %lld bytes given, %lld needed",
                  workspace_bytes, wsz);
  }

  const Span sq = span("q", q, ntok * Dk * es), sk = span("k", k, ntok * Dk * es),
             sv = span("v", v, ntok * Dv * es), sg = span("gate", gate, ngate * 4),
             sb = span("beta", beta, ntok * 4), sh0 = span("h0", h0, nst * 4),
             so = span("o", o, T > 0 ? ntok * Dv * es : 0), shT = span("hT", hT, nst * 4);
  for (const Span& in : {sq, sk, sv, sg, sb, sh0, shT})
    if (overlap(so, in)) return fail(LA_EINVAL, "o overlaps %s", in.name);
  const Span sw = span("workspace", workspace, wsz);
  for (const Span& in : {sq, sk, sv, sg, sb, sh0, so, shT})
    if (overlap(sw, in)) return fail(LA_EINVAL, "workspace overlaps %s", in.name);
  for (const Span& in : {sq, sk, sv, sg, sb})
    if (overlap(shT, in)) return fail(LA_EINVAL, "hT overlaps %s", in.name);
  if (hT && h0 && hT != h0 && overlap(shT, sh0))
    return fail(LA_EINVAL, "hT partially overlaps h0 (only hT == h0 is allowed)");
  if (int rc = check_gate_affine(gsc, gbi, H, o, T > 0 ? ntok * Dv * es : 0, hT, nst * 4,
                                 workspace, wsz))
    return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) {
    if (!hT || hT == h0) return ok();
    return hip_status(la::launch_state_init(h0, hT, nst, st), "state init launch");
  }
  const int logit = gate_mode == LA_GATE_BOUNDED_LOGIT;
  if (channel)
    return hip_status(la::launch_chunk_fwd_channel(q, k, v, gate, logit, G, beta, h0, o, hT, B,
                                                   T, H, Dk, Dv, dtype == LA_FP32, workspace,
                                                   st),
                      "chunk_fwd_channel launch");
  hipError_t e = dtype == LA_FP32
      ? la::launch_chunk_fwd(q, k, v, gate, logit, G, beta, h0, o, hT, B, T, H, Dk, Dv, raw, st,
                             gsc, gbi)
      : la::launch_chunk_fwd_pair(q, k, v, gate, logit, G, beta, h0, o, hT, B, T, H, Dk, Dv,
                                  raw, workspace, st, gsc, gbi);
  return hip_status(e, "chunk_fwd launch");
}

}  // namespace

extern "C" {

int lin_attn_chunk_fwd(const void* q, const void* k, const void* v, const float* gate,
                       int gate_mode, float G, const float* beta, const float* h0, void* o,
                       float* hT, int B, int T, int H, int Dk, int Dv, int dtype,
                       void* workspace, long long workspace_bytes, void* stream) {
  return chunk_fwd(q, k, v, gate, gate_mode, G, beta, h0, o, hT, B, T, H, Dk, Dv, dtype,
                   workspace, workspace_bytes, stream, 0);
}

int lin_attn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* gate,
                               int gate_mode, float G, const float* beta, const float* h0,
                               void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                               int dtype, void* stream) {
  if (int rc = check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return rc;
  const long long need = chunk_workspace(B, T, H, Dk, Dv, dtype);
  if (need > la::kNoAllocScratchBytes)
    return fail(LA_EINVAL,
                "these sizes need %lld bytes of scratch; lin_attn_chunk_fwd_noalloc holds at "
                "most %lld (use lin_attn_chunk_fwd with a workspace)",
                need, la::kNoAllocScratchBytes);
  void* scratch = nullptr;
  if (need > 0 && B > 0 && H > 0) {
    if (int rc = hip_status(la::noalloc_scratch(&scratch), "scratch address")) return rc;
  }
  return chunk_fwd(q, k, v, gate, gate_mode, G, beta, h0, o, hT, B, T, H, Dk, Dv, dtype,
                   scratch, scratch ? la::kNoAllocScratchBytes : 0, stream, 0);
}

long long lin_attn_chunk_fwd_channel_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                   int dtype) {
  if (check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return -1;
  ok();
  return channel_workspace(B, T, H, Dk, Dv, dtype);
}

int lin_attn_chunk_fwd_channel(const void* q, const void* k, const void* v, const float* gate,
                               int gate_mode, float G, const float* beta, const float* h0,
                               void* o, float* hT, int B, int T, int H, int Dk, int Dv,
                               int dtype, void* workspace, long long workspace_bytes,
                               void* stream) {
  return chunk_fwd(q, k, v, gate, gate_mode, G, beta, h0, o, hT, B, T, H, Dk, Dv, dtype,
                   workspace, workspace_bytes, stream, 0, 1);
}

int lin_attn_chunk_fwd_raw(const void* q, const void* k, const void* v, const float* gate,
                           int gate_mode, float G, const float* beta_logit, const float* h0,
                           void* o, float* hT, int B, int T, int H, int Dk, int Dv, int dtype,
                           void* workspace, long long workspace_bytes, void* stream) {
  return chunk_fwd(q, k, v, gate, gate_mode, G, beta_logit, h0, o, hT, B, T, H, Dk, Dv, dtype,
                   workspace, workspace_bytes, stream, 1);
}

int lin_attn_chunk_fwd_raw_affine(const void* q, const void* k, const void* v,
                                  const float* gate_x, float G, const float* gate_scale,
                                  const float* gate_bias, const float* beta_logit,
                                  const float* h0, void* o, float* hT, int B, int T, int H,
                                  int Dk, int Dv, int dtype, void* workspace,
                                  long long workspace_bytes, void* stream) {
  return chunk_fwd(q, k, v, gate_x, LA_GATE_BOUNDED_LOGIT, G, beta_logit, h0, o, hT, B, T, H, Dk,
                   Dv, dtype, workspace, workspace_bytes, stream, 1, 0, gate_scale, gate_bias);
}

long long lin_attn_chunk_fwd_varlen_workspace_size(int T, int nseq, int H, int Dk, int Dv,
                                                   int dtype) {
  if (check_varlen_sizes(T, nseq, H, Dk, Dv, dtype)) return -1;
  ok();
  // the fp32 path needs no workspace
  return dtype == LA_BF16 ? la::chunk_pair_varlen_workspace_bytes(T, nseq, H) : 0;
}

}  // extern "C"

namespace {

// lin_attn_chunk_fwd_varlen (raw = 0) and lin_attn_chunk_fwd_varlen_raw (raw = 1).
int chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* gate,
                     int gate_mode, float G, const float* beta, const float* h0, void* o,
                     float* hT, const int* cu_seqlens, int nseq, int T, int H, int Dk, int Dv,
                     int dtype, void* workspace, long long workspace_bytes, void* stream,
                     int raw, const float* gsc = nullptr, const float* gbi = nullptr) {
  if (int rc = check_varlen_sizes(T, nseq, H, Dk, Dv, dtype)) return rc;
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  // the fp32 path needs no workspace
  const long long wsz = dtype == LA_BF16 ? la::chunk_pair_varlen_workspace_bytes(T, nseq, H) : 0;
  if (nseq == 0 || H == 0) return ok();
  const int64_t es = dtype == LA_BF16 ? 2 : 4;
  const int64_t ntok = (int64_t)T * H;
  const int64_t nst = (int64_t)nseq * H * Dk * Dv;
  if (!cu_seqlens) return fail(LA_EINVAL, "cu_seqlens must not be NULL");
  if (!aligned(cu_seqlens, 4u)) return fail(LA_EINVAL, "cu_seqlens must be 4-byte aligned");
  if (T > 0) {
    const struct { const char* nm; const void* p; unsigned a; } req[] = {
        {"q", q, 16u}, {"k", k, 16u}, {"v", v, 16u}, {"gate", gate, 4u}, {"beta", beta, 4u},
        {"o", o, dtype == LA_BF16 ? 8u : 4u}};
    for (const auto& r : req) {
      if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
      if (!aligned(r.p, r.a)) return fail(LA_EINVAL, "%s must be %u-byte aligned", r.nm, r.a);
    }
  }
  if (h0 && !aligned(h0, 4u)) return fail(LA_EINVAL, "h0 must be 4-byte aligned");
  if (hT && !aligned(hT, 4u)) return fail(LA_EINVAL, "hT must be 4-byte aligned");
  if (wsz > 0) {
    if (!workspace) return fail(LA_EINVAL, "workspace must not be NULL (%lld bytes needed)", wsz);
    if (!aligned(workspace, 256u)) return fail(LA_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < wsz)
      return fail(LA_EINVAL, "workspace too small: %lld bytes given, %lld needed",
                  workspace_bytes, wsz);
  }
  const Span sq = span("q", q, ntok * Dk * es), sk = span("k", k, ntok * Dk * es),
             sv = span("v", v, ntok * Dv * es), sg = span("gate", gate, ntok * 4),
             sb = span("beta", beta, ntok * 4), sh0 = span("h0", h0, nst * 4),
             so = span("o", o, ntok * Dv * es), shT = span("hT", hT, nst * 4),
             sc = span("cu_seqlens", cu_seqlens, ((int64_t)nseq + 1) * 4);
  for (const Span& in : {sq, sk, sv, sg, sb, sh0, shT, sc})
    if (overlap(so, in)) return fail(LA_EINVAL, "o overlaps %s", in.name);
  const Span sw = span("workspace", workspace, wsz);
  for (const Span& in : {sq, sk, sv, sg, sb, sh0, so, shT, sc})
    if (overlap(sw, in)) return fail(LA_EINVAL, "workspace overlaps %s", in.name);
  for (const Span& in : {sq, sk, sv, sg, sb, sc})
    if (overlap(shT, in)) return fail(LA_EINVAL, "hT overlaps %s", in.name);
  if (hT && h0 && hT != h0 && overlap(shT, sh0))
    return fail(LA_EINVAL, "hT partially overlaps h0 (only hT == h0 is allowed)");
  if (int rc = check_gate_affine(gsc, gbi, H, o, ntok * Dv * es, hT, nst * 4, workspace, wsz))
    return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e =
      dtype == LA_BF16
          ? la::launch_chunk_fwd_pair_varlen(q, k, v, gate, gate_mode == LA_GATE_BOUNDED_LOGIT, G,
                                             beta, h0, o, hT, cu_seqlens, nseq, T, H, Dk, Dv, raw,
                                             workspace, st, gsc, gbi)
          : la::launch_chunk_fwd_varlen(q, k, v, gate, gate_mode == LA_GATE_BOUNDED_LOGIT, G, beta,
                                        h0, o, hT, cu_seqlens, nseq, T, H, Dk, Dv, raw, st, gsc,
                                        gbi);
  return hip_status(e, "chunk_fwd_varlen launch");
}

}  // namespace

extern "C" {

}  // extern "C"

namespace {

int check_channel_varlen_sizes(int T, int nseq, int H, int Dk, int Dv, int dtype) {
  if (nseq < 0) return fail(LA_EINVAL, "nseq must be >= 0, got %d", nseq);
  if (int rc = check_chunk_sizes(nseq > 0 ? 1 : 0, T, H, Dk, Dv, dtype)) return rc;
  if ((int64_t)nseq * H * (Dv / 16) > INT32_MAX || (int64_t)T / 16 + nseq + 1 > INT32_MAX / 2)
    return fail(LA_EINVAL, "problem too large (nseq = %d)", nseq);
  return LA_OK;
}

// lin_attn_chunk_fwd_channel_varlen: the per-channel gate over packed sequences.
int chunk_fwd_channel_varlen(const void* q, const void* k, const void* v, const float* gate,
                             int gate_mode, float G, const float* beta, const float* h0, void* o,
                             float* hT, const int* cu_seqlens, int nseq, int T, int H, int Dk,
                             int Dv, int dtype, void* workspace, long long workspace_bytes,
                             void* stream) {
  if (int rc = check_channel_varlen_sizes(T, nseq, H, Dk, Dv, dtype)) return rc;
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  if (G > 10.f)
    return fail(LA_ERANGE, "G must be in [0, 10] for a per-channel gate, got %g", (double)G);
  const long long wsz = la::chunk_channel_varlen_workspace_bytes(T, nseq, H, Dk, dtype == LA_FP32);
  if (nseq == 0 || H == 0) return ok();
  const int64_t es = dtype == LA_BF16 ? 2 : 4;
  const int64_t ntok = (int64_t)T * H;
  const int64_t nst = (int64_t)nseq * H * Dk * Dv;
  if (!cu_seqlens) return fail(LA_EINVAL, "cu_seqlens must not be NULL");
  if (!aligned(cu_seqlens, 4u)) return fail(LA_EINVAL, "cu_seqlens must be 4-byte aligned");
  if (T > 0) {
    const struct { const char* nm; const void* p; unsigned a; } req[] = {
        {"q", q, 16u}, {"k", k, 16u}, {"v", v, 16u}, {"gate", gate, 16u}, {"beta", beta, 4u},
        {"o", o, dtype == LA_BF16 ? 8u : 4u}};
    for (const auto& r : req) {
      if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
      if (!aligned(r.p, r.a)) return fail(LA_EINVAL, "%s must be %u-byte aligned", r.nm, r.a);
    }
  }
  if (h0 && !aligned(h0, 4u)) return fail(LA_EINVAL, "h0 must be 4-byte aligned");
  if (hT && !aligned(hT, 4u)) return fail(LA_EINVAL, "hT must be 4-byte aligned");
  if (!workspace) return fail(LA_EINVAL, "workspace must not be NULL (%lld bytes needed)", wsz);
  if (!aligned(workspace, 256u)) return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < wsz)
    return fail(LA_EINVAL, "workspace too small: %lld bytes given, %lld needed", workspace_bytes,
                wsz);
  const Span sq = span("q", q, ntok * Dk * es), sk = span("k", k, ntok * Dk * es),
             sv = span("v", v, ntok * Dv * es), sg = span("gate", gate, ntok * Dk * 4),
             sb = span("beta", beta, ntok * 4), sh0 = span("h0", h0, nst * 4),
             so = span("o", o, ntok * Dv * es), shT = span("hT", hT, nst * 4),
             sc = span("cu_seqlens", cu_seqlens, ((int64_t)nseq + 1) * 4);
  for (const Span& in : {sq, sk, sv, sg, sb, sh0, shT, sc})
    if (overlap(so, in)) return fail(LA_EINVAL, "o overlaps %s", in.name);
  const Span sw = span("workspace", workspace, wsz);
  for (const Span& in : {sq, sk, sv, sg, sb, sh0, so, shT, sc})
    if (overlap(sw, in)) return fail(LA_EINVAL, "workspace overlaps %s", in.name);
  for (const Span& in : {sq, sk, sv, sg, sb, sc})
    if (overlap(shT, in)) return fail(LA_EINVAL, "hT overlaps %s", in.name);
  if (hT && h0 && hT != h0 && overlap(shT, sh0))
    return fail(LA_EINVAL, "hT partially overlaps h0 (only hT == h0 is allowed)");
  hipError_t e = la::launch_chunk_fwd_channel_varlen(
      q, k, v, gate, gate_mode == LA_GATE_BOUNDED_LOGIT, G, beta, h0, o, hT, cu_seqlens, nseq, T,
      H, Dk, Dv, dtype == LA_FP32, workspace, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "chunk_fwd_channel_varlen launch");
}

}  // namespace

extern "C" {

long long lin_attn_chunk_fwd_channel_varlen_workspace_size(int T, int nseq, int H, int Dk,
                                                           int Dv, int dtype) {
  if (check_channel_varlen_sizes(T, nseq, H, Dk, Dv, dtype)) return -1;
  ok();
  return la::chunk_channel_varlen_workspace_bytes(T, nseq, H, Dk, dtype == LA_FP32);
}

int lin_attn_chunk_fwd_channel_varlen(const void* q, const void* k, const void* v,
                                      const float* gate, int gate_mode, float G,
                                      const float* beta, const float* h0, void* o, float* hT,
                                      const int* cu_seqlens, int nseq, int T, int H, int Dk,
                                      int Dv, int dtype, void* workspace,
                                      long long workspace_bytes, void* stream) {
  return chunk_fwd_channel_varlen(q, k, v, gate, gate_mode, G, beta, h0, o, hT, cu_seqlens, nseq,
                                  T, H, Dk, Dv, dtype, workspace, workspace_bytes, stream);
}

int lin_attn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* gate,
                              int gate_mode, float G, const float* beta, const float* h0,
                              void* o, float* hT, const int* cu_seqlens, int nseq, int T, int H,
                              int Dk, int Dv, int dtype, void* workspace,
                              long long workspace_bytes, void* stream) {
  return chunk_fwd_varlen(q, k, v, gate, gate_mode, G, beta, h0, o, hT, cu_seqlens, nseq, T, H,
                          Dk, Dv, dtype, workspace, workspace_bytes, stream, 0);
}

int lin_attn_chunk_fwd_varlen_raw(const void* q, const void* k, const void* v, const float* gate,
                                  int gate_mode, float G, const float* beta_logit,
                                  const float* h0, void* o, float* hT, const int* cu_seqlens,
                                  int nseq, int T, int H, int Dk, int Dv, int dtype,
                                  void* workspace, long long workspace_bytes, void* stream) {
  return chunk_fwd_varlen(q, k, v, gate, gate_mode, G, beta_logit, h0, o, hT, cu_seqlens, nseq,
                          T, H, Dk, Dv, dtype, workspace, workspace_bytes, stream, 1);
}

int lin_attn_chunk_fwd_varlen_raw_affine(const void* q, const void* k, const void* v,
                                         const float* gate_x, float G, const float* gate_scale,
                                         const float* gate_bias, const float* beta_logit,
                                         const float* h0, void* o, float* hT,
                                         const int* cu_seqlens, int nseq, int T, int H, int Dk,
                                         int Dv, int dtype, void* workspace,
                                         long long workspace_bytes, void* stream) {
  return chunk_fwd_varlen(q, k, v, gate_x, LA_GATE_BOUNDED_LOGIT, G, beta_logit, h0, o, hT,
                          cu_seqlens, nseq, T, H, Dk, Dv, dtype, workspace, workspace_bytes,
                          stream, 1, gate_scale, gate_bias);
}

}  // extern "C"

namespace {

// lin_attn_decode_step (channel = 0) and lin_attn_decode_step_channel (1).
int decode_step(const void* q, const void* k, const void* v, const float* gate, int gate_mode,
                float G, const float* beta, float* S, void* o, int B, int H, int Dk, int Dv,
                int dtype, void* stream, int channel) {
  if (B < 0 || H < 0) return fail(LA_EINVAL, "sizes must be >= 0 (B=%d H=%d)", B, H);
  if (dtype != LA_BF16 && dtype != LA_FP32)
    return fail(LA_EINVAL, "dtype must be LA_BF16 (0) or LA_FP32 (1), got %d", dtype);
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  if ((Dk != 64 && Dk != 128) || (Dv != 64 && Dv != 128))
    return fail(LA_EUNSUPPORTED, "decode supports Dk, Dv in {64, 128}, got Dk=%d Dv=%d", Dk, Dv);
  if ((int64_t)B * H > INT32_MAX) return fail(LA_EINVAL, "B*H exceeds 2^31");
  if (B == 0 || H == 0) return ok();
  const int64_t es = dtype == LA_BF16 ? 2 : 4;
  // S is read and written as 16-byte vectors; everything else element-wise
  const struct { const char* nm; const void* p; unsigned a; } req[] = {
      {"q", q, (unsigned)es}, {"k", k, (unsigned)es}, {"v", v, (unsigned)es},
      {"gate", gate, 4u}, {"beta", beta, 4u}, {"S", S, 16u}, {"o", o, (unsigned)es}};
  if (channel && G > 10.f)
    return fail(LA_ERANGE, "G must be in [0, 10] for a per-channel gate, got %g", (double)G);
  for (const auto& r : req) {
    if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
    if (!aligned(r.p, r.a)) return fail(LA_EINVAL, "%s must be %u-byte aligned", r.nm, r.a);
  }
  const int64_t bh = (int64_t)B * H;
  const Span sq = span("q", q, bh * Dk * es), sk = span("k", k, bh * Dk * es),
             sv = span("v", v, bh * Dv * es), sg = span("gate", gate, bh * (channel ? Dk : 1) * 4),
             sb = span("beta", beta, bh * 4), sS = span("S", S, bh * Dk * Dv * 4),
             so = span("o", o, bh * Dv * es);
  for (const Span& in : {sq, sk, sv, sg, sb, sS})
    if (overlap(so, in)) return fail(LA_EINVAL, "o overlaps %s", in.name);
  for (const Span& in : {sq, sk, sv, sg, sb})
    if (overlap(sS, in)) return fail(LA_EINVAL, "S overlaps %s", in.name);
  hipError_t e = (channel ? la::launch_decode_channel : la::launch_decode)(
      q, k, v, gate, gate_mode == LA_GATE_BOUNDED_LOGIT, G, beta, S, o, (int)bh, Dk, Dv,
      dtype == LA_FP32, reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "decode launch");
}

}  // namespace

extern "C" {

int lin_attn_decode_step(const void* q, const void* k, const void* v, const float* gate,
                         int gate_mode, float G, const float* beta, float* S, void* o, int B,
                         int H, int Dk, int Dv, int dtype, void* stream) {
  return decode_step(q, k, v, gate, gate_mode, G, beta, S, o, B, H, Dk, Dv, dtype, stream, 0);
}

int lin_attn_decode_step_channel(const void* q, const void* k, const void* v, const float* gate,
                                 int gate_mode, float G, const float* beta, float* S, void* o,
                                 int B, int H, int Dk, int Dv, int dtype, void* stream) {
  return decode_step(q, k, v, gate, gate_mode, G, beta, S, o, B, H, Dk, Dv, dtype, stream, 1);
}

long long lin_attn_chunk_bwd_workspace_size(int B, int T, int H, int Dk, int Dv, int dtype) {
  if (check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return -1;
  if ((int64_t)B * H * ((T + 15) / 16) > INT32_MAX) {
    fail(LA_EINVAL, "problem too large (B*H*T/16 exceeds 2^31)");
    return -1;
  }
  ok();
  return la::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, dtype == LA_FP32);
}

static int chunk_bwd_call(const void* q, const void* k, const void* v, const float* gate,
                          int gate_mode, float G, const float* beta, const float* h0,
                       const void* dout, const float* dhT, float* dq, float* dk, float* dv,
                       float* dgate, float* dbeta, float* dh0, int B, int T, int H, int Dk,
                       int Dv, int dtype, void* workspace, long long workspace_bytes,
                       void* stream, int seg) {
  if (int rc = check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return rc;
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  if ((int64_t)B * H * ((T + 15) / 16) > INT32_MAX)
    return fail(LA_EINVAL, "problem too large (B*H*T/16 exceeds 2^31)");
  if (B == 0 || H == 0) return ok();
  const int64_t es = dtype == LA_BF16 ? 2 : 4;
  const int64_t ntok = (int64_t)B * T * H;
  const int64_t nst = (int64_t)B * H * Dk * Dv;
  const long long wsz =
      T == 0 ? 0
      : seg  ? la::chunk_bwd_bf16_segmented_workspace_bytes(T, H, Dk, Dv, seg)
             : la::chunk_bwd_workspace_bytes(B, T, H, Dk, Dv, dtype == LA_FP32);
  if (T > 0) {
    // q, k are read and dq, dk, dv written in 16-byte vectors of a row;
    // everything else element-wise
    const struct { const char* nm; const void* p; unsigned a; } req[] = {
        {"q", q, 16u}, {"k", k, 16u}, {"v", v, (unsigned)es}, {"gate", gate, 4u},
        {"beta", beta, 4u}, {"dout", dout, (unsigned)es}, {"dq", dq, 16u}, {"dk", dk, 16u},
        {"dv", dv, 16u}, {"dgate", dgate, 4u}, {"dbeta", dbeta, 4u}};
    for (const auto& r : req) {
      if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
      if (!aligned(r.p, r.a)) return fail(LA_EINVAL, "%s must be %u-byte aligned", r.nm, r.a);
    }
    if (!workspace) return fail(LA_EINVAL, "workspace must not be NULL (%lld bytes needed)", wsz);
    if (!aligned(workspace, 256u)) return fail(LA_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < wsz)
      return fail(LA_EINVAL, "workspace too small: %lld bytes given, %lld needed",
                  workspace_bytes, wsz);
  }
  for (const auto& r : {std::make_pair("h0", (const void*)h0), std::make_pair("dhT", (const void*)dhT),
                        std::make_pair("dh0", (const void*)dh0)})
    if (r.second && !aligned(r.second, 4u)) return fail(LA_EINVAL, "%s must be 4-byte aligned", r.first);
  const int64_t tk = T > 0 ? ntok : 0;
  const Span ins[] = {span("q", q, tk * Dk * es),      span("k", k, tk * Dk * es),
                      span("v", v, tk * Dv * es),      span("gate", gate, tk * 4),
                      span("beta", beta, tk * 4),      span("h0", h0, nst * 4),
                      span("dout", dout, tk * Dv * es), span("dhT", dhT, nst * 4)};
  const Span outs[] = {span("dq", dq, tk * Dk * 4),    span("dk", dk, tk * Dk * 4),
                       span("dv", dv, tk * Dv * 4),    span("dgate", dgate, tk * 4),
                       span("dbeta", dbeta, tk * 4),   span("dh0", dh0, nst * 4),
                       span("workspace", workspace, wsz)};
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
    for (const Span& in : ins)
      if (overlap(outs[i], in)) return fail(LA_EINVAL, "%s overlaps %s", outs[i].name, in.name);
    for (size_t j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(LA_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (T == 0) {
    if (!dh0) return ok();
    return hip_status(la::launch_state_init(dhT, dh0, nst, st), "state init launch");
  }
  const hipError_t e =
      seg ? la::launch_chunk_bwd_bf16_segmented(q, k, v, dout, gate,
                                                gate_mode == LA_GATE_BOUNDED_LOGIT, G, beta, h0,
                                                dhT, dq, dk, dv, dgate, dbeta, dh0, B, T, H, Dk,
                                                Dv, seg, workspace, st)
          : la::launch_chunk_bwd(q, k, v, dout, gate, gate_mode == LA_GATE_BOUNDED_LOGIT, G,
                                 beta, h0, dhT, dq, dk, dv, dgate, dbeta, dh0, B, T, H, Dk, Dv,
                                 dtype == LA_FP32, workspace, st);
  return hip_status(e, "chunk_bwd launch");
}

int lin_attn_chunk_bwd(const void* q, const void* k, const void* v, const float* gate,
                       int gate_mode, float G, const float* beta, const float* h0,
                       const void* dout, const float* dhT, float* dq, float* dk, float* dv,
                       float* dgate, float* dbeta, float* dh0, int B, int T, int H, int Dk,
                       int Dv, int dtype, void* workspace, long long workspace_bytes,
                       void* stream) {
  return chunk_bwd_call(q, k, v, gate, gate_mode, G, beta, h0, dout, dhT, dq, dk, dv, dgate,
                        dbeta, dh0, B, T, H, Dk, Dv, dtype, workspace, workspace_bytes, stream, 0);
}

// The segmented form is for the bf16 matrix-core path with segments of whole
// groups of four tiles.
static int check_segment(int T, int H, int Dk, int Dv, int dtype, int segment_tokens) {
  if (!la::chunk_bwd_bf16_path(Dk, Dv, dtype == LA_FP32))
    return fail(LA_EINVAL, "segmented reverse pass needs dtype LA_BF16, Dk 64 or 128 and Dv <= 128");
  if (segment_tokens <= 0 || segment_tokens % 64 != 0)
    return fail(LA_EINVAL, "segment_tokens must be a positive multiple of 64 (got %d)",
                segment_tokens);
  if ((int64_t)H * ((std::min(T, segment_tokens) + 15) / 16) > INT32_MAX)
    return fail(LA_EINVAL, "segment too large (H*segment_tokens/16 exceeds 2^31)");
  return LA_OK;
}

long long lin_attn_chunk_bwd_segmented_workspace_size(int B, int T, int H, int Dk, int Dv,
                                                      int dtype, int segment_tokens) {
  if (check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return -1;
  if (check_segment(T, H, Dk, Dv, dtype, segment_tokens)) return -1;
  ok();
  return T > 0 ? la::chunk_bwd_bf16_segmented_workspace_bytes(T, H, Dk, Dv, segment_tokens) : 0;
}

int lin_attn_chunk_bwd_segmented(const void* q, const void* k, const void* v, const float* gate,
                                 int gate_mode, float G, const float* beta, const float* h0,
                                 const void* dout, const float* dhT, float* dq, float* dk,
                                 float* dv, float* dgate, float* dbeta, float* dh0, int B, int T,
                                 int H, int Dk, int Dv, int dtype, int segment_tokens,
                                 void* workspace, long long workspace_bytes, void* stream) {
  if (int rc = check_chunk_sizes(B, T, H, Dk, Dv, dtype)) return rc;
  if (int rc = check_segment(T, H, Dk, Dv, dtype, segment_tokens)) return rc;
  return chunk_bwd_call(q, k, v, gate, gate_mode, G, beta, h0, dout, dhT, dq, dk, dv, dgate,
                        dbeta, dh0, B, T, H, Dk, Dv, dtype, workspace, workspace_bytes, stream,
                        segment_tokens);
}

long long lin_attn_chunk_bwd_varlen_workspace_size(int T, int nseq, int H, int Dk, int Dv,
                                                   int dtype) {
  if (check_varlen_sizes(T, nseq, H, Dk, Dv, dtype)) return -1;
  if ((int64_t)H * (T / 16 + nseq + 1) > INT32_MAX) {
    fail(LA_EINVAL, "problem too large (H*(T/16+nseq+1) exceeds 2^31)");
    return -1;
  }
  ok();
  return la::chunk_bwd_varlen_workspace_bytes(T, nseq, H, Dk, Dv, dtype == LA_FP32);
}

int lin_attn_chunk_bwd_varlen(const void* q, const void* k, const void* v, const float* gate,
                              int gate_mode, float G, const float* beta, const float* h0,
                              const void* dout, const float* dhT, float* dq, float* dk,
                              float* dv, float* dgate, float* dbeta, float* dh0,
                              const int* cu_seqlens, int nseq, int T, int H, int Dk, int Dv,
                              int dtype, void* workspace, long long workspace_bytes,
                              void* stream) {
  if (int rc = check_varlen_sizes(T, nseq, H, Dk, Dv, dtype)) return rc;
  if (int rc = check_gate_scalars(gate_mode, G)) return rc;
  if ((int64_t)H * (T / 16 + nseq + 1) > INT32_MAX)
    return fail(LA_EINVAL, "problem too large (H*(T/16+nseq+1) exceeds 2^31)");
  if (nseq == 0 || H == 0) return ok();
  if (!cu_seqlens) return fail(LA_EINVAL, "cu_seqlens must not be NULL");
  if (!aligned(cu_seqlens, 4u)) return fail(LA_EINVAL, "cu_seqlens must be 4-byte aligned");
  const int64_t es = dtype == LA_BF16 ? 2 : 4;
  const int64_t ntok = (int64_t)T * H;
  const int64_t nst = (int64_t)nseq * H * Dk * Dv;
  const long long wsz = la::chunk_bwd_varlen_workspace_bytes(T, nseq, H, Dk, Dv, dtype == LA_FP32);
  if (T > 0) {
    // q, k are read and dq, dk, dv written in 16-byte vectors of a row;
    // everything else element-wise
    const struct { const char* nm; const void* p; unsigned a; } req[] = {
        {"q", q, 16u}, {"k", k, 16u}, {"v", v, (unsigned)es}, {"gate", gate, 4u},
        {"beta", beta, 4u}, {"dout", dout, (unsigned)es}, {"dq", dq, 16u}, {"dk", dk, 16u},
        {"dv", dv, 16u}, {"dgate", dgate, 4u}, {"dbeta", dbeta, 4u}};
    for (const auto& r : req) {
      if (!r.p) return fail(LA_EINVAL, "%s must not be NULL", r.nm);
      if (!aligned(r.p, r.a)) return fail(LA_EINVAL, "%s must be %u-byte aligned", r.nm, r.a);
    }
  }
  for (const auto& r : {std::make_pair("h0", (const void*)h0), std::make_pair("dhT", (const void*)dhT),
                        std::make_pair("dh0", (const void*)dh0)})
    if (r.second && !aligned(r.second, 4u)) return fail(LA_EINVAL, "%s must be 4-byte aligned", r.first);
  if (!workspace) return fail(LA_EINVAL, "workspace must not be NULL (%lld bytes needed)", wsz);
  if (!aligned(workspace, 256u)) return fail(LA_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < wsz)
    return fail(LA_EINVAL, "workspace too small: %lld bytes given, %lld needed", workspace_bytes,
                wsz);
  const Span ins[] = {span("q", q, ntok * Dk * es),      span("k", k, ntok * Dk * es),
                      span("v", v, ntok * Dv * es),      span("gate", gate, ntok * 4),
                      span("beta", beta, ntok * 4),      span("h0", h0, nst * 4),
                      span("dout", dout, ntok * Dv * es), span("dhT", dhT, nst * 4),
                      span("cu_seqlens", cu_seqlens, ((int64_t)nseq + 1) * 4)};
  const Span outs[] = {span("dq", dq, ntok * Dk * 4),    span("dk", dk, ntok * Dk * 4),
                       span("dv", dv, ntok * Dv * 4),    span("dgate", dgate, ntok * 4),
                       span("dbeta", dbeta, ntok * 4),   span("dh0", dh0, nst * 4),
                       span("workspace", workspace, wsz)};
  for (size_t i = 0; i < sizeof outs / sizeof outs[0]; ++i) {
    for (const Span& in : ins)
      if (overlap(outs[i], in)) return fail(LA_EINVAL, "%s overlaps %s", outs[i].name, in.name);
    for (size_t j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(LA_EINVAL, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  hipError_t e = la::launch_chunk_bwd_varlen(
      q, k, v, dout, gate, gate_mode == LA_GATE_BOUNDED_LOGIT, G, beta, h0, dhT, dq, dk, dv, dgate,
      dbeta, dh0, cu_seqlens, nseq, T, H, Dk, Dv, dtype == LA_FP32, workspace,
      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e, "chunk_bwd_varlen launch");
}

int lin_attn_gate(const float* x, float G, float* g, long long n, void* stream) {
  if (n < 0) return fail(LA_EINVAL, "n must be >= 0, got %lld", n);
  if (!std::isfinite(G) || G < 0.f || G > 16.f)
    return fail(LA_ERANGE, "G must be finite and in [0, 16], got %g", (double)G);
  if (n == 0) return ok();
  if (!x || !g) return fail(LA_EINVAL, "x and g must not be NULL");
  if (!aligned(x, 4u) || !aligned(g, 4u)) return fail(LA_EINVAL, "x and g must be 4-byte aligned");
  if (x != g && overlap(span("x", x, n * 4), span("g", g, n * 4)))
    return fail(LA_EINVAL, "g partially overlaps x (only g == x is allowed)");
  return hip_status(la::launch_gate(x, G, g, n, reinterpret_cast<hipStream_t>(stream)),
                    "gate launch");
}

}  // extern "C"
