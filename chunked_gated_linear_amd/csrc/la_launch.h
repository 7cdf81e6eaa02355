// la_launch.h -- internal launchers behind the C ABI (include/lin_attn.h).
// Arguments are already validated by the caller; each returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

namespace la {

// fp32 path: one fused kernel, no workspace.  raw != 0: q and k are
// L2-normalised per token inside the pass and beta holds logits.  gsc, gbi
// (the forward launchers, logit mode): per-head scale and shift of the gate
// logit, NULL for 1 and 0.
hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v,
                            const float* gate, int gate_logit, float G,
                            const float* beta, const float* h0, void* o, float* hT,
                            int B, int T, int H, int Dk, int Dv, int raw, hipStream_t st,
                            const float* gsc = nullptr, const float* gbi = nullptr);

// The fp32 path over packed sequences: sequence s is tokens [cu[s], cu[s+1])
// of one packed sequence of T tokens (cu: device array of nseq + 1 offsets).
hipError_t launch_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                   const float* gate, int gate_logit, float G,
                                   const float* beta, const float* h0, void* o, float* hT,
                                   const int* cu, int nseq, int T, int H, int Dk, int Dv,
                                   int raw, hipStream_t st, const float* gsc = nullptr,
                                   const float* gbi = nullptr);

// bf16 path: intra-tile kernel into the workspace, then the inter-tile kernel;
// the state is carried across pairs of 16-token tiles.  raw != 0: q and k are
// L2-normalised per token inside the pass and beta holds logits.
hipError_t launch_chunk_fwd_pair(const void* q, const void* k, const void* v,
                                 const float* gate, int gate_logit, float G,
                                 const float* beta, const float* h0, void* o, float* hT,
                                 int B, int T, int H, int Dk, int Dv, int raw, void* ws,
                                 hipStream_t st, const float* gsc = nullptr,
                                 const float* gbi = nullptr);

// Workspace bytes the bf16 path needs (0 when T == 0): one record per pair of
// tiles and head, plus one fp32 state per head for sequences long enough to be
// cut into stretches.
long long chunk_pair_workspace_bytes(int B, int T, int H, int Dk, int Dv);

// Packed sequences (bf16): sequence s is tokens [cu[s], cu[s+1]) of one packed
// sequence of T tokens; cu is a device array of nseq + 1 offsets.
hipError_t launch_chunk_fwd_pair_varlen(const void* q, const void* k, const void* v,
                                        const float* gate, int gate_logit, float G,
                                        const float* beta, const float* h0, void* o, float* hT,
                                        const int* cu, int nseq, int T, int H, int Dk, int Dv,
                                        int raw, void* ws, hipStream_t st,
                                        const float* gsc = nullptr, const float* gbi = nullptr);

// Workspace bytes of the packed-sequence path: H * (T / 32 + nseq + 1) records.
long long chunk_pair_varlen_workspace_bytes(int T, int nseq, int H);

// Reverse mode over 16-token tiles (fp32 arithmetic; q, k, v, dout bf16 or
// fp32 as `fp32` says): gradients of q, k, v, the gate (g, or its logit when
// gate_logit), beta and h0.  dhT and h0 may be NULL (zeros); dh0 may be NULL.
hipError_t launch_chunk_bwd(const void* q, const void* k, const void* v, const void* dout,
                            const float* gate, int gate_logit, float G, const float* beta,
                            const float* h0, const float* dhT, float* dq, float* dk, float* dv,
                            float* dgate, float* dbeta, float* dh0, int B, int T, int H, int Dk,
                            int Dv, int fp32, void* ws, hipStream_t st);

// Workspace bytes of the reverse pass: per tile and head a 3200-byte record
// and, for float32 inputs (or d_v > 128), the fp32 state at the tile start and
// the fp32 gradient of its end state; for bf16 inputs the state only at every
// second tile and the gradient at every fourth, as packed bf16 hi / lo words.
long long chunk_bwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int fp32);

// The reverse pass over packed sequences: sequence s is tokens
// [cu[s], cu[s+1]) of one packed sequence of T tokens (cu: device array of
// B + 1 offsets); its tiles take per-head slots floor(cu[s] / 16) + s + c.
hipError_t launch_chunk_bwd_varlen(const void* q, const void* k, const void* v, const void* dout,
                                   const float* gate, int gate_logit, float G, const float* beta,
                                   const float* h0, const float* dhT, float* dq, float* dk,
                                   float* dv, float* dgate, float* dbeta, float* dh0,
                                   const int* cu, int B, int T, int H, int Dk, int Dv, int fp32,
                                   void* ws, hipStream_t st);

// Workspace bytes of the packed reverse pass: H * (T / 16 + nseq + 1) tiles,
// each as in chunk_bwd_workspace_bytes.
long long chunk_bwd_varlen_workspace_bytes(int T, int nseq, int H, int Dk, int Dv, int fp32);

// The reverse pass for bf16 inputs on the bf16 matrix cores (chunk_bwd_bf16.hip),
// taken by launch_chunk_bwd / launch_chunk_bwd_varlen whenever
// chunk_bwd_bf16_path says so: states kept at every second tile and state
// gradients at every fourth as packed bf16 hi / lo words, the tiles between
// rebuilt in the gradient kernel.  cu == NULL: B sequences of T tokens; else
// B packed sequences.
bool chunk_bwd_bf16_path(int Dk, int Dv, int fp32);
long long chunk_bwd_bf16_workspace_bytes(int B, int T, int H, int Dk, int Dv);
long long chunk_bwd_bf16_varlen_workspace_bytes(int T, int nseq, int H, int Dk, int Dv);
hipError_t launch_chunk_bwd_bf16(const void* q, const void* k, const void* v, const void* dout,
                                 const float* gate, int gate_logit, float G, const float* beta,
                                 const float* h0, const float* dhT, float* dq, float* dk,
                                 float* dv, float* dgate, float* dbeta, float* dh0, const int* cu,
                                 int B, int T, int H, int Dk, int Dv, void* ws, hipStream_t st);
// The same in segments of L tokens (L a multiple of 64; batched sequences):
// a forward pass keeps the states at segment starts, then each segment runs
// the reverse pass from its start state with the state gradient carried from
// the segment after it.  Workspace: one segment's, plus per head (S + 1)
// float32 states.
long long chunk_bwd_bf16_segmented_workspace_bytes(int T, int H, int Dk, int Dv, int L);
hipError_t launch_chunk_bwd_bf16_segmented(const void* q, const void* k, const void* v,
                                           const void* dout, const float* gate, int gate_logit,
                                           float G, const float* beta, const float* h0,
                                           const float* dhT, float* dq, float* dk, float* dv,
                                           float* dgate, float* dbeta, float* dh0, int B, int T,
                                           int H, int Dk, int Dv, int L, void* ws,
                                           hipStream_t st);

// Per-channel gate (gate [B, T, H, Dk]); q, k, v, o bf16 or fp32 as `fp32`
// says: a parallel tile-preparation kernel into the workspace, then the
// serial kernel (fp32 MFMA throughout for fp32 inputs; bf16 MFMA for the
// state products, hi/lo for U, for bf16 inputs).
hipError_t launch_chunk_fwd_channel(const void* q, const void* k, const void* v,
                                    const float* gate, int gate_logit, float G,
                                    const float* beta, const float* h0, void* o, float* hT,
                                    int B, int T, int H, int Dk, int Dv, int fp32, void* ws,
                                    hipStream_t st);

// The same over packed sequences: sequence s is tokens [cu[s], cu[s+1]) of one
// packed sequence of T tokens (cu: device array of nseq + 1 offsets).
hipError_t launch_chunk_fwd_channel_varlen(const void* q, const void* k, const void* v,
                                           const float* gate, int gate_logit, float G,
                                           const float* beta, const float* h0, void* o,
                                           float* hT, const int* cu, int nseq, int T, int H,
                                           int Dk, int Dv, int fp32, void* ws, hipStream_t st);

// Workspace bytes of the packed per-channel path: H * (T / 16 + nseq + 1) records.
long long chunk_channel_varlen_workspace_bytes(int T, int nseq, int H, int Dk, int fp32);

// Workspace bytes of the per-channel path: one record per tile (or pair) and
// head, and the carried state of long sequences.
long long chunk_channel_workspace_bytes(int B, int T, int H, int Dk, int Dv, int fp32);

// The per-channel path for bf16 inputs with the state stepped over 32-token
// pairs of tiles (cu == nullptr: B sequences of T tokens; else B = nseq packed
// sequences); workspace bytes of its records, batched and packed.
hipError_t launch_chunk_fwd_channel_pair(const void* q, const void* k, const void* v,
                                         const float* gate, int gate_logit, float G,
                                         const float* beta, const float* h0, void* o, float* hT,
                                         int B, int T, int H, int Dk, int Dv, const int* cu,
                                         void* ws, hipStream_t st);
long long chunk_channel_pair_workspace_bytes(int B, int T, int H, int Dk, int Dv);
long long chunk_channel_pair_varlen_workspace_bytes(int T, int nseq, int H, int Dk);

// Decode step with a per-channel gate (gate [B*H, Dk]), state in place.
hipError_t launch_decode_channel(const void* q, const void* k, const void* v,
                                 const float* gate, int gate_logit, float G, const float* beta,
                                 float* S, void* o, int BH, int Dk, int Dv, int fp32,
                                 hipStream_t st);

hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* gate, int gate_logit, float G,
                         const float* beta, float* S, void* o, int BH, int Dk,
                         int Dv, int fp32, hipStream_t st);

hipError_t launch_gate(const float* x, float G, float* g, long long n, hipStream_t st);

// Compute units of the current device, queried once per device and then
// served from a per-device cache (the count never changes while the process
// runs); 256 if the query fails.
int device_cus();

// Range check of a forward pass's inputs (the caller synchronises): flags[0]
// gets bit 1 for a non-finite q, k or v element, bit 2 for a gate value
// outside [-G, 0] or non-finite (log mode) or NaN (logit mode), bit 4 for a
// beta outside [0, 1] or non-finite, bit 8 for a non-finite h0 element.
// flags must hold one unsigned int; it is cleared first.
hipError_t launch_range_check(const void* q, const void* k, const void* v, const float* gate,
                              int gate_logit, float G, const float* beta, const float* h0,
                              long long nqk, long long nv, long long ngate, long long nbeta,
                              long long nh0, int fp32, unsigned* flags, hipStream_t st);

// Size of the library-owned scratch of lin_attn_chunk_fwd_noalloc (one copy
// per GPU), and its device address on the current device, resolved with
// hipGetSymbolAddress on first use per device.
constexpr long long kNoAllocScratchBytes = 64ll << 20;
hipError_t noalloc_scratch(void** ptr);

// hT <- h0 (or zeros when h0 is NULL), n floats.
hipError_t launch_state_init(const float* h0, float* hT, long long n, hipStream_t st);

}  // namespace la
