// kdn_kernels.h -- host-side launchers of the libkdn kernels (internal).
// Plain host declarations: the C ABI (kdn_api.cpp) needs only these, so it
// also builds with a host compiler alone (the sanitizer test does that).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kdn {

// Optional timing of the next kernel launched through launch_k: the dispatch
// itself records the start and stop events (hipExtLaunchKernel), so that no
// marker packet sits between the kernels.  Per host thread; consumed by that
// one launch.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchTiming& launch_timing();

// A packed batch of N variable-length sequences: every head's rows hold the
// sequences one after another ([H][Ttot][d]); sequence s has rows
// cu[s]..cu[s+1] and its chunks are numbered from cc[s] (cc[s] = sum over the
// earlier sequences of ceil(length / chunk)).  Device pointers.
struct Packed {
    const int32_t* cu = nullptr;
    const int32_t* cc = nullptr;
    int H = 1;
    int Ttot = 0;
};

struct Shape {
    int BH;  // B * H (heads, or sequences * heads for decode and packed batches)
    int T;   // tokens per head (packed: total tokens per head)
    int dk, dv, chunk;
    int nc;  // ceil(T / chunk) (packed: the longest sequence's chunk count)
    bool diag;
    bool qkv_bf16, gate_bf16, gain_bf16;
    bool varlen = false;  // a packed batch (pk), BH = N * H
    Packed pk;
};

// Each launcher returns hipSuccess or the launch error.  Pointers are device
// pointers with the layouts documented in include/kdn.h.

// Moebius products the scan keeps per (chunk, precision): for the diagonal
// variant the prefix products of the chunk's tokens after every 16 tokens
// (16, 32, ..., the last one being the chunk's product), which the prep pass
// starts its 16-token sub-blocks from; for the isotropic variant the chunk's
// product alone.
inline int agg_subs(const Shape& s) { return s.diag ? s.chunk / 16 : 1; }

// Moebius scan, pass 1: per-chunk products of the 2x2 token matrices.
// agg: [BH][nc][agg_subs][nl] float4 (nl = dk for diagonal, 1 for isotropic);
// entry s of a chunk is the product of its first 16 (s + 1) tokens (later
// tokens on the left), the last entry the chunk's whole product.
hipError_t launch_scan_reduce(const Shape& s, const void* k, const void* a, const void* nu,
                              const void* r, float* agg, hipStream_t st);
// Offsets of a packed batch (cu_in: the caller's N + 1 sequence offsets):
// a sanitised copy cu and the chunk offsets cc, both N + 1 int32.
hipError_t launch_packed_table(const int32_t* cu_in, int N, int Ttot, int C, int32_t* cu,
                               int32_t* cc, hipStream_t st);
// Moebius scan, pass 2: chunk-boundary precisions lam_chunk [BH][nc+1][nl] and
// lambda_T [BH][nl] (either may be NULL) from lambda0 (NULL -> ones).
hipError_t launch_scan_carry(const Shape& s, const float* agg, const float* lambda0,
                             float* lam_chunk, float* lambda_T, hipStream_t st);
// Moebius scan, pass 3: per-token predictive precision lambda_minus
// [BH][T][nl] from the chunk-boundary values.
hipError_t launch_scan_emit(const Shape& s, const void* k, const void* a, const void* nu,
                            const void* r, const float* lam_chunk, float* lambda_minus,
                            hipStream_t st);
// Kalman gain from given predictive precisions; w [BH][T][dk] in gain dtype.
hipError_t launch_gain(const Shape& s, const void* k, const void* r, const float* lambda_minus,
                       void* w, hipStream_t st);
// Per-chunk preparation: optionally the gain (from lam_chunk, written to w),
// then A = strict_tril(K W^T * Gamma) and T = (I + A)^{-1} written to Tm
// [BH][nc][chunk][chunk] in qkv dtype, and the chunk-local cumulative log2
// decay g [BH][nc][chunk] (float32).  fuse_gain = false reads w instead.
// dinv (diagonal, fused gain; may be NULL): 1 / (k^T P^- k + r) per token
// [BH][T] (float32), kept for the backward pass.
// agg (the scan's products; may be NULL without the fused gain): each
// 16-token sub-block of a diagonal chunk starts from the chunk-boundary
// precision carried through the prefix product before it.
hipError_t launch_chunk_prep(const Shape& s, bool fuse_gain, const void* k, const void* a,
                             const void* nu, const void* r, const float* lam_chunk,
                             const float* agg, void* w, void* Tm, float* g, hipStream_t st,
                             float* dinv = nullptr);
// Workspace of a state pass over sequence segments: nseg segments per head
// (state_split), the start state of every segment
// Sseg [BH][nseg][dv][dk] and the linear part of every segment's affine map
// Aseg [BH][nseg][dk][dk], both float32.
struct SegWs {
    int nseg = 1, Lc = 0, L0 = 0;  // L0: chunks of segment 0 (0: Lc)
    float* Sseg = nullptr;
    float* Aseg = nullptr;
};
// How the state pass cuts each head's chunks for this shape: nseg segments
// (1: the plain sequential pass), the first of L0 chunks, the others of Lc.
struct SegSplit {
    int nseg, Lc, L0;
};
SegSplit state_split(const Shape& s);
// Sequential chunk pass: memory write and read-out (g from the prep pass).
// Sc (may be NULL): the state at every chunk start, [BH][nc][dv][dk] in qkv
// dtype, kept for the backward pass.
// o may be NULL (not written) when only Sc is wanted.
// seg (may be NULL): with seg->nseg > 1 (and o given, Sc NULL, a fixed-length
// batch) the pass runs over sequence segments in three launches: each
// segment's affine map, their composition in order, and the read-out of every
// segment from its start state.
hipError_t launch_chunk_state(const Shape& s, const void* q, const void* k, const void* v,
                              const float* g, const void* w, const void* Tm, const float* S0,
                              void* o, float* S_T, hipStream_t st, void* Sc = nullptr,
                              const SegWs* seg = nullptr);
// One decode step in place.  slot (may be NULL): per active sequence, the
// cache slot of its state among n_slots (H heads each); outside [0, n_slots):
// idle, nothing read or written for that sequence.
hipError_t launch_decode(const Shape& s, const void* q, const void* k, const void* v,
                         const void* a, const void* nu, const void* r, float* S, float* lam,
                         void* o, hipStream_t st, const int32_t* slot = nullptr, int H = 1,
                         int n_slots = 0);

// Backward pass (diagonal variant).  Device pointers; per-token arrays are
// [BH][T], per-(token, dim) arrays [BH][T][d], per-chunk states [BH][nc][dv][dk].
struct BwdArgs {
    const void *q, *k, *v, *a, *nu, *r;  // the forward's inputs
    const void* dO;                      // [BH][T][dv], qkv dtype
    const float *dS_T, *dlambda_T;       // may be NULL (zero)
    const void *w, *Tm;                  // the forward's gain keys and T matrices
    const float *g, *lam_chunk, *dinv;   // log2 decays, boundary precisions, 1/D
    const void* Sc;                      // state at every chunk start (qkv dtype)
    void* dSe;                           // state adjoint at every chunk end (qkv dtype)
    void* dW;                            // dW [BH][T][dk], qkv dtype
    float *sdot, *dlna;                  // s_t and d(ln a_t) [BH][T]
    float *ab, *Gout;                    // per (chunk, dim): float2 map, G at the chunk end
    float *dq, *dk, *dv, *da, *dnu, *dr;  // outputs
    float *dlambda0, *dS0;               // outputs, may be NULL
};
// reverse state pass: dv, dSe, dS0
hipError_t launch_bwd_state(const Shape& s, const BwdArgs& b, hipStream_t st);
// per-chunk gradients: dq, dk (memory part), dW, sdot, dlna
hipError_t launch_bwd_grad(const Shape& s, const BwdArgs& b, hipStream_t st);
// gain and precision recursion: dk (+= gain part), da, dnu, dr, dlambda0
hipError_t launch_bwd_gain(const Shape& s, const BwdArgs& b, hipStream_t st);
bool backward_supported(const Shape& s);

// Exact KDN gain (dense Riccati recursion) per token; P0 [BH][dk][dk] or NULL
// (identity); w [BH][T][dk] in qkv dtype; P_T [BH][dk][dk] or NULL.
hipError_t launch_dense_gain(const Shape& s, const void* k, const void* a, const void* nu,
                             const void* r, const float* P0, void* w, float* P_T,
                             hipStream_t st);

// true if the chunk kernels are built for this (dtype, dk, dv, chunk)
bool chunk_supported(const Shape& s);
bool decode_supported(const Shape& s);

}  // namespace kdn
