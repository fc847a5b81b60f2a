// kdn_api.cpp -- the C ABI of libkdn (declared in include/kdn.h): descriptor
// validation, workspace layout and the order in which the kernels run.
//
// kdn_forward runs four kernels on the caller's stream:
//   1. scan reduce   per-chunk products of the 2x2 Moebius matrices
//   2. scan carry    chunk-boundary precisions and lambda_T
//   3. chunk prep    gain w of every token (from the boundary precision) and
//                    T = (I + A)^{-1} of every chunk, all chunks in parallel
//   4. chunk state   sequential pass per (head, d_v tile): innovations, memory
//                    write and read-out on MFMA
// Workspace (all offsets 256-byte aligned): Moebius aggregates, boundary
// precisions, gain keys w, the per-chunk T matrices and the chunk-local
// cumulative log2 decays.
#include "kdn.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>
#include <climits>

#include "kdn_kernels.h"

namespace kdn {
LaunchTiming& launch_timing() {
    static thread_local LaunchTiming t;
    return t;
}
}  // namespace kdn

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == KDN_BF16 ? 2 : 4; }

kdn_status check_common(const kdn_desc* d) {
    if (!d) return KDN_ERR_NULL;
    if (d->B < 0 || d->H < 0 || d->d_k < 0 || d->d_v < 0) return KDN_ERR_SHAPE;
    if (d->variant != KDN_DIAGONAL && d->variant != KDN_ISOTROPIC) return KDN_ERR_UNSUPPORTED;
    for (int t : {d->qkv_dtype, d->gate_dtype, d->gain_dtype})
        if (t != KDN_F32 && t != KDN_BF16) return KDN_ERR_UNSUPPORTED;
    if (!dim_ok(d->d_k) || !dim_ok(d->d_v)) return KDN_ERR_UNSUPPORTED;
    if ((int64_t)d->B * d->H > INT32_MAX) return KDN_ERR_UNSUPPORTED;
    return KDN_OK;
}

kdn_status check_chunked(const kdn_desc* d) {
    kdn_status s = check_common(d);
    if (s != KDN_OK) return s;
    if (d->T < 0 || d->chunk < 0) return KDN_ERR_SHAPE;
    if (d->chunk != 16 && d->chunk != 32 && d->chunk != 64) return KDN_ERR_UNSUPPORTED;
    if ((int64_t)d->B * d->H > 65535) return KDN_ERR_UNSUPPORTED;  // heads index grid.y
    return KDN_OK;
}

kdn::Shape make_shape(const kdn_desc* d) {
    kdn::Shape s;
    s.BH = d->B * d->H;
    s.T = d->T > 0 ? d->T : 0;
    s.dk = d->d_k;
    s.dv = d->d_v;
    s.chunk = d->chunk > 0 ? d->chunk : 1;
    s.nc = (d->T + s.chunk - 1) / s.chunk;
    s.diag = d->variant == KDN_DIAGONAL;
    s.qkv_bf16 = d->qkv_dtype == KDN_BF16;
    s.gate_bf16 = d->gate_dtype == KDN_BF16;
    s.gain_bf16 = d->gain_dtype == KDN_BF16;
    return s;
}

struct ForwardWs {
    size_t agg, lam_chunk, w, tm, g, seg_S, seg_A, total;
    int nseg, Lc, L0;
};

// workspace offsets: [agg | lam_chunk | w | T | g | segment states | segment
// maps]; kdn_chunk_delta uses [T | g].  The segment arrays are empty unless
// the state pass runs over sequence segments (few heads, many chunks).
ForwardWs forward_ws(const kdn_desc* d) {
    const kdn::Shape s = make_shape(d);
    const size_t nl = s.diag ? s.dk : 1;
    ForwardWs w;
    const kdn::SegSplit sp = kdn::chunk_supported(s) ? kdn::state_split(s)
                                                     : kdn::SegSplit{1, s.nc, s.nc};
    w.nseg = sp.nseg > 1 ? sp.nseg : 1;
    w.Lc = w.nseg > 1 ? sp.Lc : s.nc;
    w.L0 = w.nseg > 1 ? sp.L0 : s.nc;
    const size_t segs = w.nseg > 1 ? (size_t)s.BH * w.nseg : 0;
    w.agg = 0;
    w.lam_chunk = w.agg + round_up((size_t)s.BH * s.nc * kdn::agg_subs(s) * nl * 16);
    w.w = w.lam_chunk + round_up((size_t)s.BH * (s.nc + 1) * nl * 4);
    w.tm = w.w + round_up((size_t)s.BH * s.T * s.dk * esize(d->qkv_dtype));
    w.g = w.tm + round_up((size_t)s.BH * s.nc * s.chunk * s.chunk * esize(d->qkv_dtype));
    w.seg_S = w.g + round_up((size_t)s.BH * s.nc * s.chunk * 4);
    w.seg_A = w.seg_S + round_up(segs * s.dv * s.dk * 4);
    w.total = w.seg_A + round_up(segs * s.dk * s.dk * 4);
    return w;
}

// backward workspace: the forward's, then [1/D | chunk-start states |
// chunk-end adjoints | dW (qkv dtype) | s | d(ln a) | chunk maps (float2) |
// G at chunk ends]
struct BackwardWs {
    ForwardWs f;
    size_t dinv, Sc, dSe, dW, sdot, dlna, ab, Gout, total;
};

BackwardWs backward_ws(const kdn_desc* d) {
    const kdn::Shape s = make_shape(d);
    BackwardWs b;
    b.f = forward_ws(d);
    const size_t n = (size_t)s.BH * s.T;
    const size_t states = (size_t)s.BH * s.nc * s.dv * s.dk * esize(d->qkv_dtype);
    const size_t per_dim = (size_t)s.BH * s.nc * (s.diag ? s.dk : 1);
    b.dinv = b.f.total;
    b.Sc = b.dinv + round_up(n * 4);
    b.dSe = b.Sc + round_up(states);
    b.dW = b.dSe + round_up(states);
    b.sdot = b.dW + round_up(n * s.dk * esize(d->qkv_dtype));
    b.dlna = b.sdot + round_up(n * 4);
    b.ab = b.dlna + round_up(n * 4);
    b.Gout = b.ab + round_up(per_dim * 8);
    b.total = b.Gout + round_up(per_dim * 4);
    return b;
}

// Packed batches: d->B sequences, d->T tokens per head in all.  The chunk
// count is bounded by sum ceil(L / C) <= (T + B (C - 1)) / C whatever the
// lengths, which sizes the per-chunk arrays.  Layout: [cu | cc | agg |
// lam_chunk | w | T | g].
struct PackedWs {
    size_t cu, cc, agg, lam_chunk, w, tm, g, seg_S, seg_A, total;
    int nc_bound, nseg_max;
};

// the segment count of the state pass for a packed batch of N sequences whose
// longest has max_chunks chunks (1: no segments)
int packed_segments(const kdn_desc* d, int max_chunks) {
    kdn::Shape s = make_shape(d);
    s.varlen = true;
    s.BH = d->B * d->H;
    s.nc = max_chunks;
    return kdn::chunk_supported(s) ? std::max(1, kdn::state_split(s).nseg) : 1;
}

// workspace offsets: [cu | cc | agg | lam_chunk | w | T | g | segment states |
// segment maps]; the segment arrays are sized for the largest segment count any
// split of the T tokens could ask for (one sequence holding them all)
PackedWs packed_ws(const kdn_desc* d) {
    const kdn::Shape s = make_shape(d);
    const size_t N = d->B > 0 ? d->B : 0, H = d->H, nl = s.diag ? s.dk : 1;
    const size_t ncb = (s.T + N * (s.chunk - 1)) / s.chunk;
    PackedWs w;
    w.nc_bound = static_cast<int>(ncb);
    w.nseg_max = N > 0 && H > 0 ? packed_segments(d, (s.T + s.chunk - 1) / s.chunk) : 1;
    const size_t segs = w.nseg_max > 1 ? N * H * w.nseg_max : 0;
    w.cu = 0;
    w.cc = round_up((N + 1) * 4);
    w.agg = w.cc + round_up((N + 1) * 4);
    w.lam_chunk = w.agg + round_up(H * ncb * kdn::agg_subs(s) * nl * 16);
    w.w = w.lam_chunk + round_up(H * (ncb + N) * nl * 4);
    w.tm = w.w + round_up(H * s.T * s.dk * esize(d->qkv_dtype));
    w.g = w.tm + round_up(H * ncb * s.chunk * s.chunk * esize(d->qkv_dtype));
    w.seg_S = w.g + round_up(H * ncb * s.chunk * 4);
    w.seg_A = w.seg_S + round_up(segs * s.dv * s.dk * 4);
    w.total = w.seg_A + round_up(segs * s.dk * s.dk * 4);
    return w;
}

kdn_status hip_status(hipError_t e) { return e == hipSuccess ? KDN_OK : KDN_ERR_HIP; }

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

}  // namespace

extern "C" {

const char* kdn_status_string(kdn_status s) {
    switch (s) {
        case KDN_OK: return "ok";
        case KDN_ERR_NULL: return "a required pointer is NULL";
        case KDN_ERR_SHAPE: return "negative or inconsistent sizes";
        case KDN_ERR_UNSUPPORTED: return "unsupported size, dtype, variant or chunk";
        case KDN_ERR_WORKSPACE: return "workspace too small";
        case KDN_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case KDN_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    }
    return "unknown kdn_status";
}

kdn_status kdn_validate(const kdn_desc* d) {
    kdn_status s = check_chunked(d);
    if (s != KDN_OK) return s;
    if (!kdn::chunk_supported(make_shape(d))) return KDN_ERR_UNSUPPORTED;
    return KDN_OK;
}

size_t kdn_forward_workspace_bytes(const kdn_desc* d) {
    if (kdn_validate(d) != KDN_OK) return 0;
    return forward_ws(d).total;
}

int32_t kdn_forward_segments(const kdn_desc* d) {
    if (kdn_validate(d) != KDN_OK) return 0;
    return forward_ws(d).nseg;
}

size_t kdn_mobius_scan_workspace_bytes(const kdn_desc* d) {
    if (check_chunked(d) != KDN_OK) return 0;
    const ForwardWs w = forward_ws(d);
    return w.w;  // aggregates + boundary precisions
}

namespace {

// The forward's kernels first..last in order, `reps` times over; with
// timing events (events NULL: none) on the kernels of one pass.
kdn_status forward_run(const kdn_desc* d, const void* q, const void* k, const void* v,
                       const void* a, const void* qnoise, const void* r, const float* lambda0,
                       const float* S0, void* o, float* S_T, float* lambda_T, void* ws,
                       size_t ws_bytes, void* stream, void* const* events, int first, int last,
                       int reps) {
    kdn_status st = kdn_validate(d);
    if (st != KDN_OK) return st;
    const kdn::Shape s = make_shape(d);
    const ForwardWs w = forward_ws(d);
    if (s.BH == 0) return KDN_OK;
    if (s.T > 0 && (!q || !k || !v || !a || !qnoise || !r || !o)) return KDN_ERR_NULL;
    if (!ws) return KDN_ERR_NULL;
    if (ws_bytes < w.total) return KDN_ERR_WORKSPACE;
    for (const void* p : {q, k, v, (const void*)o, (const void*)S0, (const void*)S_T, (const void*)ws})
        if (p && !aligned16(p)) return KDN_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    float* agg = reinterpret_cast<float*>(at(ws, w.agg));
    float* lc = reinterpret_cast<float*>(at(ws, w.lam_chunk));
    void* wk = at(ws, w.w);
    void* tm = at(ws, w.tm);
    float* g = reinterpret_cast<float*>(at(ws, w.g));
    // timing: the dispatches themselves record the start and stop events of
    // each kernel (entries may be NULL)
    auto timed = [&](int i) {
        kdn::LaunchTiming t;
        if (events) {
            t.start = static_cast<hipEvent_t>(events[2 * i]);
            t.stop = static_cast<hipEvent_t>(events[2 * i + 1]);
        }
        kdn::launch_timing() = t;
    };
    kdn::Shape sw = s;
    sw.gain_bf16 = s.qkv_bf16;
    kdn::SegWs seg;
    seg.nseg = w.nseg;
    seg.Lc = w.Lc;
    seg.L0 = w.L0;
    seg.Sseg = reinterpret_cast<float*>(at(ws, w.seg_S));
    seg.Aseg = reinterpret_cast<float*>(at(ws, w.seg_A));
    auto launch = [&](int i) -> hipError_t {
        switch (i) {
            case 0: return kdn::launch_scan_reduce(s, k, a, qnoise, r, agg, hs);
            case 1: return kdn::launch_scan_carry(s, agg, lambda0, lc, lambda_T, hs);
            case 2: return kdn::launch_chunk_prep(sw, true, k, a, qnoise, r, lc, agg, wk, tm, g, hs);
            default:
                return kdn::launch_chunk_state(s, q, k, v, g, wk, tm, S0, o, S_T, hs, nullptr, &seg);
        }
    };
    hipError_t e = hipSuccess;
    for (int rep = 0; rep < reps && e == hipSuccess; ++rep)
        for (int i = first; i <= last && e == hipSuccess; ++i) {
            timed(i);
            e = launch(i);
        }
    kdn::launch_timing() = kdn::LaunchTiming{};
    return hip_status(e);
}

}  // namespace

kdn_status kdn_forward_events(const kdn_desc* d, const void* q, const void* k, const void* v,
                              const void* a, const void* qnoise, const void* r,
                              const float* lambda0, const float* S0, void* o, float* S_T,
                              float* lambda_T, void* ws, size_t ws_bytes, void* stream,
                              void* const* events) {
    return forward_run(d, q, k, v, a, qnoise, r, lambda0, S0, o, S_T, lambda_T, ws, ws_bytes,
                       stream, events, 0, 3, 1);
}

kdn_status kdn_forward_repeat(const kdn_desc* d, const void* q, const void* k, const void* v,
                              const void* a, const void* qnoise, const void* r,
                              const float* lambda0, const float* S0, void* o, float* S_T,
                              float* lambda_T, void* ws, size_t ws_bytes, void* stream,
                              int32_t first, int32_t last, int32_t reps) {
    if (first < 0 || last > 3 || first > last || reps < 0) return KDN_ERR_SHAPE;
    // a repeated launch must read what the first one read
    if ((S_T && S0 && S_T == S0) || (lambda_T && lambda0 && lambda_T == lambda0))
        return KDN_ERR_SHAPE;
    return forward_run(d, q, k, v, a, qnoise, r, lambda0, S0, o, S_T, lambda_T, ws, ws_bytes,
                       stream, nullptr, first, last, reps);
}

size_t kdn_backward_workspace_bytes(const kdn_desc* d) {
    if (check_chunked(d) != KDN_OK) return 0;
    if (!kdn::backward_supported(make_shape(d))) return 0;
    return backward_ws(d).total;
}

}  // extern "C"

namespace {

// The backward, with (recompute) or without (the intermediates kept in ws by
// kdn_forward_keep) its forward recompute.  With keep_o, only the forward
// runs, writing o, S_T and lambda_T as well.
kdn_status backward_impl(const kdn_desc* d, const void* q, const void* k, const void* v,
                         const void* a, const void* qnoise, const void* r, const float* lambda0,
                         const float* S0, const void* dO, const float* dS_T,
                         const float* dlambda_T, float* dq, float* dk, float* dv, float* da,
                         float* dqnoise, float* dr, float* dlambda0, float* dS0, void* ws,
                         size_t ws_bytes, void* stream, void* const* events, bool recompute,
                         void* o, float* S_T, float* lambda_T) {
    const bool fwd_only = o != nullptr;
    kdn_status st = check_chunked(d);
    if (st != KDN_OK) return st;
    const kdn::Shape s = make_shape(d);
    if (!kdn::backward_supported(s)) return KDN_ERR_UNSUPPORTED;
    const BackwardWs w = backward_ws(d);
    if (s.BH == 0) return KDN_OK;
    if (s.T > 0 && (!q || !k || !v || !a || !qnoise || !r))
        return KDN_ERR_NULL;
    if (s.T > 0 && !fwd_only && (!dO || !dq || !dk || !dv || !da || !dqnoise || !dr))
        return KDN_ERR_NULL;
    if (!ws) return KDN_ERR_NULL;
    if (ws_bytes < w.total) return KDN_ERR_WORKSPACE;
    for (const void* p : {q, k, v, dO, (const void*)S0, (const void*)dS_T, (const void*)dq,
                          (const void*)dk, (const void*)dv, (const void*)dS0, (const void*)ws,
                          (const void*)o,
                          (const void*)S_T})
        if (p && !aligned16(p)) return KDN_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    float* agg = reinterpret_cast<float*>(at(ws, w.f.agg));
    float* lc = reinterpret_cast<float*>(at(ws, w.f.lam_chunk));
    void* wk = at(ws, w.f.w);
    void* tm = at(ws, w.f.tm);
    float* g = reinterpret_cast<float*>(at(ws, w.f.g));
    float* dinv = reinterpret_cast<float*>(at(ws, w.dinv));
    kdn::BwdArgs b;
    b.q = q; b.k = k; b.v = v; b.a = a; b.nu = qnoise; b.r = r;
    b.dO = dO; b.dS_T = dS_T; b.dlambda_T = dlambda_T;
    b.w = wk; b.Tm = tm; b.g = g; b.lam_chunk = lc; b.dinv = dinv;
    b.Sc = at(ws, w.Sc);
    b.dSe = at(ws, w.dSe);
    b.dW = at(ws, w.dW);
    b.sdot = reinterpret_cast<float*>(at(ws, w.sdot));
    b.dlna = reinterpret_cast<float*>(at(ws, w.dlna));
    b.ab = reinterpret_cast<float*>(at(ws, w.ab));
    b.Gout = reinterpret_cast<float*>(at(ws, w.Gout));
    b.dq = dq; b.dk = dk; b.dv = dv; b.da = da; b.dnu = dqnoise; b.dr = dr;
    b.dlambda0 = dlambda0; b.dS0 = dS0;
    auto timed = [&](int i) {
        kdn::LaunchTiming t;
        if (events) {
            t.start = static_cast<hipEvent_t>(events[2 * i]);
            t.stop = static_cast<hipEvent_t>(events[2 * i + 1]);
        }
        kdn::launch_timing() = t;
    };
    hipError_t e = hipSuccess;
    if (recompute) {
        // the forward, keeping 1/D of every token and the chunk-start states
        // (the read-out only when asked for)
        timed(0);
        e = kdn::launch_scan_reduce(s, k, a, qnoise, r, agg, hs);
        timed(1);
        if (e == hipSuccess) e = kdn::launch_scan_carry(s, agg, lambda0, lc, lambda_T, hs);
        kdn::Shape sw = s;
        sw.gain_bf16 = s.qkv_bf16;
        timed(2);
        if (e == hipSuccess)
            e = kdn::launch_chunk_prep(sw, true, k, a, qnoise, r, lc, agg, wk, tm, g, hs, dinv);
        timed(3);
        if (e == hipSuccess)
            e = kdn::launch_chunk_state(s, q, k, v, g, wk, tm, S0, o, S_T, hs, at(ws, w.Sc));
        if (fwd_only) {
            kdn::launch_timing() = kdn::LaunchTiming{};
            return hip_status(e);
        }
    }
    timed(4);
    if (e == hipSuccess) e = kdn::launch_bwd_state(s, b, hs);
    timed(5);
    if (e == hipSuccess) e = kdn::launch_bwd_grad(s, b, hs);
    timed(6);
    if (e == hipSuccess) e = kdn::launch_bwd_gain(s, b, hs);
    kdn::launch_timing() = kdn::LaunchTiming{};
    return hip_status(e);
}

}  // namespace

extern "C" {

kdn_status kdn_backward_events(const kdn_desc* d, const void* q, const void* k, const void* v,
                               const void* a, const void* qnoise, const void* r,
                               const float* lambda0, const float* S0, const void* dO,
                               const float* dS_T, const float* dlambda_T, float* dq, float* dk,
                               float* dv, float* da, float* dqnoise, float* dr, float* dlambda0,
                               float* dS0, void* ws, size_t ws_bytes, void* stream,
                               void* const* events) {
    return backward_impl(d, q, k, v, a, qnoise, r, lambda0, S0, dO, dS_T, dlambda_T, dq, dk, dv,
                         da, dqnoise, dr, dlambda0, dS0, ws, ws_bytes, stream, events, true,
                         nullptr, nullptr, nullptr);
}

kdn_status kdn_forward_keep(const kdn_desc* d, const void* q, const void* k, const void* v,
                            const void* a, const void* qnoise, const void* r,
                            const float* lambda0, const float* S0, void* o, float* S_T,
                            float* lambda_T, void* ws, size_t ws_bytes, void* stream) {
    if (d && d->T > 0 && !o) return KDN_ERR_NULL;
    if (d && d->T == 0) {
        // nothing to keep: the plain forward copies the state through
        return kdn_forward(d, q, k, v, a, qnoise, r, lambda0, S0, o, S_T, lambda_T, ws,
                           ws_bytes, stream);
    }
    return backward_impl(d, q, k, v, a, qnoise, r, lambda0, S0, nullptr, nullptr, nullptr,
                         nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         ws, ws_bytes, stream, nullptr, true, o, S_T, lambda_T);
}

kdn_status kdn_backward_kept_events(const kdn_desc* d, const void* q, const void* k,
                                    const void* v, const void* a, const void* qnoise,
                                    const void* r, const float* lambda0, const float* S0,
                                    const void* dO, const float* dS_T, const float* dlambda_T,
                                    float* dq, float* dk, float* dv, float* da, float* dqnoise,
                                    float* dr, float* dlambda0, float* dS0, void* ws,
                                    size_t ws_bytes, void* stream, void* const* events) {
    return backward_impl(d, q, k, v, a, qnoise, r, lambda0, S0, dO, dS_T, dlambda_T, dq, dk, dv,
                         da, dqnoise, dr, dlambda0, dS0, ws, ws_bytes, stream, events, false,
                         nullptr, nullptr, nullptr);
}

kdn_status kdn_backward_kept(const kdn_desc* d, const void* q, const void* k, const void* v,
                             const void* a, const void* qnoise, const void* r,
                             const float* lambda0, const float* S0, const void* dO,
                             const float* dS_T, const float* dlambda_T, float* dq, float* dk,
                             float* dv, float* da, float* dqnoise, float* dr, float* dlambda0,
                             float* dS0, void* ws, size_t ws_bytes, void* stream) {
    return kdn_backward_kept_events(d, q, k, v, a, qnoise, r, lambda0, S0, dO, dS_T, dlambda_T,
                                    dq, dk, dv, da, dqnoise, dr, dlambda0, dS0, ws, ws_bytes,
                                    stream, nullptr);
}

kdn_status kdn_backward(const kdn_desc* d, const void* q, const void* k, const void* v,
                        const void* a, const void* qnoise, const void* r, const float* lambda0,
                        const float* S0, const void* dO, const float* dS_T,
                        const float* dlambda_T, float* dq, float* dk, float* dv, float* da,
                        float* dqnoise, float* dr, float* dlambda0, float* dS0, void* ws,
                        size_t ws_bytes, void* stream) {
    return kdn_backward_events(d, q, k, v, a, qnoise, r, lambda0, S0, dO, dS_T, dlambda_T, dq,
                               dk, dv, da, dqnoise, dr, dlambda0, dS0, ws, ws_bytes, stream,
                               nullptr);
}

kdn_status kdn_forward(const kdn_desc* d, const void* q, const void* k, const void* v,
                       const void* a, const void* qnoise, const void* r, const float* lambda0,
                       const float* S0, void* o, float* S_T, float* lambda_T, void* ws,
                       size_t ws_bytes, void* stream) {
    return kdn_forward_events(d, q, k, v, a, qnoise, r, lambda0, S0, o, S_T, lambda_T, ws,
                              ws_bytes, stream, nullptr);
}

kdn_status kdn_mobius_scan(const kdn_desc* d, const void* k, const void* a, const void* qnoise,
                           const void* r, const float* lambda0, float* lambda_minus,
                           float* lambda_chunk, float* lambda_T, void* ws, size_t ws_bytes,
                           void* stream) {
    kdn_status st = check_chunked(d);
    if (st != KDN_OK) return st;
    const kdn::Shape s = make_shape(d);
    const ForwardWs w = forward_ws(d);
    if (s.BH == 0) return KDN_OK;
    if (s.T > 0 && (!k || !a || !qnoise || !r)) return KDN_ERR_NULL;
    if (!ws) return KDN_ERR_NULL;
    if (ws_bytes < w.w) return KDN_ERR_WORKSPACE;
    if (!aligned16(ws) || (k && !aligned16(k))) return KDN_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    float* agg = reinterpret_cast<float*>(at(ws, w.agg));
    float* lc = lambda_chunk ? lambda_chunk : reinterpret_cast<float*>(at(ws, w.lam_chunk));
    hipError_t e = kdn::launch_scan_reduce(s, k, a, qnoise, r, agg, hs);
    if (e == hipSuccess) e = kdn::launch_scan_carry(s, agg, lambda0, lc, lambda_T, hs);
    if (e == hipSuccess && lambda_minus)
        e = kdn::launch_scan_emit(s, k, a, qnoise, r, lc, lambda_minus, hs);
    return hip_status(e);
}

kdn_status kdn_gain(const kdn_desc* d, const void* k, const void* r, const float* lambda_minus,
                    void* w, void* stream) {
    kdn_status st = check_common(d);
    if (st != KDN_OK) return st;
    if (d->T < 0) return KDN_ERR_SHAPE;
    const kdn::Shape s = make_shape(d);
    if ((size_t)s.BH * s.T == 0) return KDN_OK;
    if (!k || !r || !lambda_minus || !w) return KDN_ERR_NULL;
    return hip_status(kdn::launch_gain(s, k, r, lambda_minus, w, static_cast<hipStream_t>(stream)));
}

size_t kdn_chunk_delta_workspace_bytes(const kdn_desc* d) {
    if (kdn_validate(d) != KDN_OK) return 0;
    const ForwardWs w = forward_ws(d);
    return w.seg_S - w.tm;  // T and g
}

kdn_status kdn_chunk_delta(const kdn_desc* d, const void* q, const void* k, const void* v,
                           const void* a, const void* w, const float* S0, void* o, float* S_T,
                           void* ws, size_t ws_bytes, void* stream) {
    kdn_status st = kdn_validate(d);
    if (st != KDN_OK) return st;
    if (d->gain_dtype != d->qkv_dtype) return KDN_ERR_UNSUPPORTED;
    if (d->d_k != 32 && d->d_k != 64 && d->d_k != 128) return KDN_ERR_UNSUPPORTED;
    const kdn::Shape s = make_shape(d);
    const ForwardWs fw = forward_ws(d);
    if (s.BH == 0) return KDN_OK;
    if (s.T > 0 && (!q || !k || !v || !a || !w || !o)) return KDN_ERR_NULL;
    if (!ws) return KDN_ERR_NULL;
    if (ws_bytes < fw.seg_S - fw.tm) return KDN_ERR_WORKSPACE;
    for (const void* p : {q, k, v, w, (const void*)o, (const void*)S0, (const void*)S_T, (const void*)ws})
        if (p && !aligned16(p)) return KDN_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    void* wk = const_cast<void*>(w);  // read only when fuse_gain is false
    float* g = reinterpret_cast<float*>(at(ws, fw.g - fw.tm));
    hipError_t e =
        kdn::launch_chunk_prep(s, false, k, a, nullptr, nullptr, nullptr, nullptr, wk, ws, g, hs);
    if (e == hipSuccess) e = kdn::launch_chunk_state(s, q, k, v, g, w, ws, S0, o, S_T, hs);
    return hip_status(e);
}

kdn_status kdn_decode_step(const kdn_desc* d, const void* q, const void* k, const void* v,
                           const void* a, const void* qnoise, const void* r, float* S,
                           float* lambda, void* o, void* stream) {
    kdn_status st = check_common(d);
    if (st != KDN_OK) return st;
    kdn::Shape s = make_shape(d);
    s.T = 1;
    s.nc = 1;
    if (s.BH == 0) return KDN_OK;
    if (!q || !k || !v || !a || !qnoise || !r || !S || !lambda || !o) return KDN_ERR_NULL;
    for (const void* p : {q, k, (const void*)S, (const void*)lambda})
        if (!aligned16(p)) return KDN_ERR_ALIGN;
    if (!kdn::decode_supported(s)) return KDN_ERR_UNSUPPORTED;
    return hip_status(kdn::launch_decode(s, q, k, v, a, qnoise, r, S, lambda, o,
                                         static_cast<hipStream_t>(stream)));
}

kdn_status kdn_dense_gain(const kdn_desc* d, const void* k, const void* a, const void* qnoise,
                          const void* r, const float* P0, void* w, float* P_T, void* stream) {
    kdn_status st = check_common(d);
    if (st != KDN_OK) return st;
    if (d->T < 0) return KDN_ERR_SHAPE;
    if (d->gain_dtype != d->qkv_dtype) return KDN_ERR_UNSUPPORTED;
    if (d->d_k != 32 && d->d_k != 64 && d->d_k != 128) return KDN_ERR_UNSUPPORTED;
    const kdn::Shape s = make_shape(d);
    if (s.BH == 0) return KDN_OK;
    if (s.T > 0 && (!k || !a || !qnoise || !r || !w)) return KDN_ERR_NULL;
    if (s.T > 0 && (!aligned16(k) || !aligned16(w))) return KDN_ERR_ALIGN;
    return hip_status(kdn::launch_dense_gain(s, k, a, qnoise, r, P0, w, P_T,
                                             static_cast<hipStream_t>(stream)));
}

size_t kdn_forward_varlen_workspace_bytes(const kdn_desc* d) {
    if (check_chunked(d) != KDN_OK) return 0;
    if (!kdn::chunk_supported(make_shape(d))) return 0;
    return packed_ws(d).total;
}

kdn_status kdn_forward_varlen(const kdn_desc* d, const int32_t* cu_seqlens, int32_t max_seqlen,
                              const void* q, const void* k, const void* v, const void* a,
                              const void* qnoise, const void* r, const float* lambda0,
                              const float* S0, void* o, float* S_T, float* lambda_T, void* ws,
                              size_t ws_bytes, void* stream) {
    kdn_status st = check_chunked(d);
    if (st != KDN_OK) return st;
    if (max_seqlen < 0) return KDN_ERR_SHAPE;
    if ((int64_t)d->B * d->H > 65535) return KDN_ERR_UNSUPPORTED;
    kdn::Shape s = make_shape(d);
    if (!kdn::chunk_supported(s)) return KDN_ERR_UNSUPPORTED;
    const PackedWs w = packed_ws(d);
    const int N = d->B;
    if (N == 0 || d->H == 0) return KDN_OK;
    if (!cu_seqlens || !ws || !S_T || !lambda_T) return KDN_ERR_NULL;
    if (s.T > 0 && (!q || !k || !v || !a || !qnoise || !r || !o)) return KDN_ERR_NULL;
    if (ws_bytes < w.total) return KDN_ERR_WORKSPACE;
    for (const void* p : {q, k, v, (const void*)o, (const void*)S0, (const void*)S_T,
                          (const void*)ws})
        if (p && !aligned16(p)) return KDN_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t* cu = reinterpret_cast<int32_t*>(at(ws, w.cu));
    int32_t* cc = reinterpret_cast<int32_t*>(at(ws, w.cc));
    // the packed batch: N * H slabs; nc is the longest sequence's chunk count
    s.varlen = true;
    s.BH = N * d->H;
    s.nc = (std::min<int32_t>(max_seqlen, s.T) + s.chunk - 1) / s.chunk;
    s.pk.cu = cu;
    s.pk.cc = cc;
    s.pk.H = d->H;
    s.pk.Ttot = s.T;
    float* agg = reinterpret_cast<float*>(at(ws, w.agg));
    float* lc = reinterpret_cast<float*>(at(ws, w.lam_chunk));
    void* wk = at(ws, w.w);
    void* tm = at(ws, w.tm);
    float* g = reinterpret_cast<float*>(at(ws, w.g));
    hipError_t e = kdn::launch_packed_table(cu_seqlens, N, s.T, s.chunk, cu, cc, hs);
    if (e == hipSuccess && s.nc > 0) e = kdn::launch_scan_reduce(s, k, a, qnoise, r, agg, hs);
    if (e == hipSuccess) e = kdn::launch_scan_carry(s, agg, lambda0, lc, lambda_T, hs);
    kdn::Shape sw = s;
    sw.gain_bf16 = s.qkv_bf16;
    if (e == hipSuccess && s.nc > 0)
        e = kdn::launch_chunk_prep(sw, true, k, a, qnoise, r, lc, agg, wk, tm, g, hs);
    // few (sequence, head) slabs over long sequences: the segmented state pass,
    // each slab cut into the same number of segments
    kdn::SegWs seg;
    seg.nseg = std::min(packed_segments(d, s.nc), w.nseg_max);
    seg.Lc = 0;  // per slab, from its own chunk count
    seg.Sseg = reinterpret_cast<float*>(at(ws, w.seg_S));
    seg.Aseg = reinterpret_cast<float*>(at(ws, w.seg_A));
    if (e == hipSuccess)
        e = kdn::launch_chunk_state(s, q, k, v, g, wk, tm, S0, o, S_T, hs, nullptr, &seg);
    return hip_status(e);
}

kdn_status kdn_decode_step_indexed(const kdn_desc* d, const void* q, const void* k,
                                   const void* v, const void* a, const void* qnoise,
                                   const void* r, float* S_cache, float* lambda_cache,
                                   const int32_t* slot, int32_t n_slots, void* o, void* stream) {
    kdn_status st = check_common(d);
    if (st != KDN_OK) return st;
    if (n_slots < 0) return KDN_ERR_SHAPE;
    kdn::Shape s = make_shape(d);
    s.T = 1;
    s.nc = 1;
    if (s.BH == 0) return KDN_OK;
    if (!q || !k || !v || !a || !qnoise || !r || !S_cache || !lambda_cache || !slot || !o)
        return KDN_ERR_NULL;
    for (const void* p : {q, k, (const void*)S_cache, (const void*)lambda_cache})
        if (!aligned16(p)) return KDN_ERR_ALIGN;
    if (!kdn::decode_supported(s)) return KDN_ERR_UNSUPPORTED;
    return hip_status(kdn::launch_decode(s, q, k, v, a, qnoise, r, S_cache, lambda_cache, o,
                                         static_cast<hipStream_t>(stream), slot, d->H,
                                         n_slots));
}

}  // extern "C"
