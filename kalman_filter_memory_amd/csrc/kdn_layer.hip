// kdn_layer.hip -- the KDN layer around the core recurrence, on caller-given
// weights ("Kalman Delta Networks", English abstract: the KDN layer is a
// drop-in replacement for linear attention in a language model; KDN summary,
// 关键模块: the layer's queries, keys, values and its three gates a, nu, r).
//
//   Z = x W_in^T                    (one library GEMM: q, k, v and the gate logits)
//   q_h, k_h = L2-normalised per head; v_h as is
//   a = sigmoid(z_a + b_a), nu = softplus(z_nu + b_nu), r = softplus(z_r + b_r)
//   o = KDN forward (kdn_forward)
//   y = concat_h(o_h) W_out^T       (one library GEMM)
//
// The weights are stored out-features major (W_in [n_in][d_model], W_out
// [d_model][H d_v], a linear layer's usual layout), so both GEMMs contract
// two operands that are contiguous along the reduction index; they run in
// hipBLASLt (fp32 accumulation), whose kernels for that layout are the fastest
// on this GPU (1.43-1.45 PFLOP/s at the layer shape against 1.16-1.21 for the
// input-major weight layout).  The normalisation, the gate activations and the
// change of layout from token rows [B*T, .] to the recurrence's per-head rows
// [B, H, T, .] are one pass (layer_in_kernel); the read-out goes back to token
// rows in another (layer_out_kernel).  Both are HBM-bound copies with 16-byte
// accesses.
#include <hipblaslt/hipblaslt.h>

#include <algorithm>
#include <mutex>
#include <new>

#include "kdn.h"
#include "kdn_device.h"

namespace {

using kdn::bf16_t;

template <typename E> struct Io;
template <> struct Io<float> {
    static constexpr int code = KDN_F32;
    static constexpr hipDataType blas = HIP_R_32F;
};
template <> struct Io<bf16_t> {
    static constexpr int code = KDN_BF16;
    static constexpr hipDataType blas = HIP_R_16BF;
};

// Device workspace of a GEMM, a slice of the layer workspace (the library
// allocates nothing per call); algorithms needing more are not chosen.
constexpr size_t kGemmWs = size_t(32) << 20;

// What kdn_blas_create returns: a hipBLASLt handle and the algorithm chosen
// for each GEMM shape seen so far (the heuristic query runs on the host once
// per shape, not per call).
struct BlasCtx {
    hipblasLtHandle_t lt = nullptr;
    std::mutex mu;
    struct Entry {
        int M, N, K, ldx, ldw, ldy;
        hipDataType type;
        hipblasLtMatmulAlgo_t algo;
    };
    Entry cache[16];
    int n = 0;
};

// N contiguous elements of E at p (16-byte aligned when N * sizeof(E) >= 16,
// else N * sizeof(E)-aligned) as floats, in vector accesses
template <typename E, int N>
__device__ __forceinline__ void load_n(const E* p, float* f) {
    constexpr int W = N * int(sizeof(E)) / 4;  // 32-bit words
    uint32_t u[W];
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int i = 0; i < W / 4; ++i) {
            const kdn::u32x4 x = reinterpret_cast<const kdn::u32x4*>(p)[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) u[4 * i + j] = x[j];
        }
    } else if constexpr (W == 2) {
        const kdn::u32x2 x = *reinterpret_cast<const kdn::u32x2*>(p);
        u[0] = x[0];
        u[1] = x[1];
    } else {
        u[0] = *reinterpret_cast<const uint32_t*>(p);
    }
#pragma unroll
    for (int i = 0; i < W; ++i) {
        if constexpr (sizeof(E) == 4) {
            f[i] = __uint_as_float(u[i]);
        } else {
            f[2 * i] = __uint_as_float(u[i] << 16);
            f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
}
template <typename E, int N>
__device__ __forceinline__ void store_n(E* p, const float* f) {
    constexpr int W = N * int(sizeof(E)) / 4;
    uint32_t u[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
        if constexpr (sizeof(E) == 4)
            u[i] = __float_as_uint(f[i]);
        else
            u[i] = uint32_t(kdn::f2bf(f[2 * i])) | (uint32_t(kdn::f2bf(f[2 * i + 1])) << 16);
    }
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int i = 0; i < W / 4; ++i)
            reinterpret_cast<kdn::u32x4*>(p)[i] =
                kdn::u32x4{u[4 * i], u[4 * i + 1], u[4 * i + 2], u[4 * i + 3]};
    } else if constexpr (W == 2) {
        *reinterpret_cast<kdn::u32x2*>(p) = kdn::u32x2{u[0], u[1]};
    } else {
        *reinterpret_cast<uint32_t*>(p) = u[0];
    }
}

// One workgroup per token row.  Each group of 16 lanes handles one vector of
// the row (q_h, k_h or v_h; d/16 elements per lane); threads below 3H apply
// the gate activations.
template <typename E, int DK, int DV>
__global__ __launch_bounds__(256) void layer_in_kernel(
    const E* __restrict__ Z, int ldz, const float* __restrict__ bg, int H, int T,
    E* __restrict__ q, E* __restrict__ k, E* __restrict__ v, E* __restrict__ a,
    E* __restrict__ nu, E* __restrict__ r) {
    const int row = blockIdx.x, b = row / T, t = row % T;
    const int tid = threadIdx.x, grp = tid >> 4, l16 = tid & 15;
    const E* z = Z + size_t(row) * ldz;
    // up to four vectors per 16-lane group at a time, every load issued before
    // the first is used
    constexpr int NK = DK / 16, NV = DV / 16, NM = NK > NV ? NK : NV, U = 4;
    for (int base = 0; base < 3 * H; base += 16 * U) {
        float xs[U][NM];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = base + grp + 16 * u;
            if (vi < 2 * H) load_n<E, NK>(z + vi * DK + l16 * NK, xs[u]);
            else if (vi < 3 * H) load_n<E, NV>(z + 2 * H * DK + (vi - 2 * H) * DV + l16 * NV, xs[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int vi = base + grp + 16 * u;
            if (vi < 2 * H) {  // q or k: x / max(|x|, 1e-6)
                const int h = vi < H ? vi : vi - H;
                float* x = xs[u];
                float ss = 0.f;
#pragma unroll
                for (int i = 0; i < NK; ++i) ss = fmaf(x[i], x[i], ss);
                ss = kdn::group_sum<16>(ss);
                const float sc = 1.f / sqrtf(fmaxf(ss, 1e-12f));
#pragma unroll
                for (int i = 0; i < NK; ++i) x[i] *= sc;
                E* dst = (vi < H ? q : k) + ((size_t(b) * H + h) * T + t) * DK + l16 * NK;
                store_n<E, NK>(dst, x);
            } else if (vi < 3 * H) {
                const int h = vi - 2 * H;
                store_n<E, NV>(v + ((size_t(b) * H + h) * T + t) * DV + l16 * NV, xs[u]);
            }
        }
    }
    if (tid < 3 * H) {
        const int g = tid / H, h = tid % H;
        const float x = kdn::to_f<E>(z[H * (2 * DK + DV) + tid]) + bg[tid];
        float y;
        if (g == 0) {
            y = 1.f / (1.f + expf(-x));
        } else {
            y = x > 20.f ? x : log1pf(expf(x));
        }
        E* dst = g == 0 ? a : g == 1 ? nu : r;
        dst[(size_t(b) * H + h) * T + t] = kdn::from_f<E>(y);
    }
}

// o [B,H,T,DV] -> token rows [B*T, H*DV], 16 bytes per thread and step
template <typename E, int DV>
__global__ __launch_bounds__(256) void layer_out_kernel(const E* __restrict__ o,
                                                        E* __restrict__ o2, int H, int T) {
    constexpr int VE = 16 / sizeof(E);  // elements per 16 bytes
    const int row = blockIdx.x, b = row / T, t = row % T;
    const int n16 = H * DV / VE;
    for (int c = threadIdx.x; c < n16; c += 256) {
        const int e = c * VE, h = e / DV, j = e % DV;
        const kdn::u32x4 x =
            *reinterpret_cast<const kdn::u32x4*>(o + ((size_t(b) * H + h) * T + t) * DV + j);
        *reinterpret_cast<kdn::u32x4*>(o2 + size_t(row) * H * DV + e) = x;
    }
}

template <typename E, int DK, int DV>
hipError_t in_t(const void* Z, int ldz, const float* bg, int M, int H, int T, void* q, void* k,
                void* v, void* a, void* nu, void* r, hipStream_t st) {
    layer_in_kernel<E, DK, DV><<<M, 256, 0, st>>>(
        static_cast<const E*>(Z), ldz, bg, H, T, static_cast<E*>(q), static_cast<E*>(k),
        static_cast<E*>(v), static_cast<E*>(a), static_cast<E*>(nu), static_cast<E*>(r));
    return hipGetLastError();
}

template <typename E>
hipError_t launch_in(int dk, int dv, const void* Z, int ldz, const float* bg, int M, int H, int T,
                     void* q, void* k, void* v, void* a, void* nu, void* r, hipStream_t st) {
#define KDN_LAYER_IN(DK_, DV_) \
    if (dk == DK_ && dv == DV_) return in_t<E, DK_, DV_>(Z, ldz, bg, M, H, T, q, k, v, a, nu, r, st);
    KDN_LAYER_IN(32, 32) KDN_LAYER_IN(32, 64) KDN_LAYER_IN(32, 128)
    KDN_LAYER_IN(64, 32) KDN_LAYER_IN(64, 64) KDN_LAYER_IN(64, 128)
    KDN_LAYER_IN(128, 32) KDN_LAYER_IN(128, 64) KDN_LAYER_IN(128, 128)
#undef KDN_LAYER_IN
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t launch_out(int dv, const void* o, void* o2, int M, int H, int T, hipStream_t st) {
#define KDN_LAYER_OUT(DV_)                                                                 \
    if (dv == DV_) {                                                                       \
        layer_out_kernel<E, DV_><<<M, 256, 0, st>>>(static_cast<const E*>(o),              \
                                                    static_cast<E*>(o2), H, T);            \
        return hipGetLastError();                                                          \
    }
    KDN_LAYER_OUT(32) KDN_LAYER_OUT(64) KDN_LAYER_OUT(128)
#undef KDN_LAYER_OUT
    return hipErrorInvalidValue;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct LayerWs {
    size_t z, q, k, v, a, nu, r, o, gemm, core, total;
    int ldz;
};

kdn_desc core_desc(const kdn_layer_desc* d) {
    kdn_desc c{};
    c.B = d->B;
    c.H = d->H;
    c.T = d->T;
    c.d_k = d->d_k;
    c.d_v = d->d_v;
    c.chunk = d->chunk;
    c.variant = d->variant;
    c.qkv_dtype = d->dtype;
    c.gate_dtype = d->dtype;
    c.gain_dtype = d->dtype;
    return c;
}

int n_in(const kdn_layer_desc* d) { return d->H * (2 * d->d_k + d->d_v) + 3 * d->H; }

LayerWs layer_ws(const kdn_layer_desc* d) {
    const size_t es = d->dtype == KDN_BF16 ? 2 : 4;
    const size_t M = size_t(d->B) * d->T, BH = size_t(d->B) * d->H;
    LayerWs w{};
    w.ldz = (n_in(d) + 15) / 16 * 16;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align256(bytes);
        return o;
    };
    // Z is dead once layer_in_kernel has run; the token-row read-out reuses it
    w.z = take(M * std::max<size_t>(w.ldz, size_t(d->H) * d->d_v) * es);
    w.q = take(BH * d->T * d->d_k * es);
    w.k = take(BH * d->T * d->d_k * es);
    w.v = take(BH * d->T * d->d_v * es);
    w.a = take(BH * d->T * es);
    w.nu = take(BH * d->T * es);
    w.r = take(BH * d->T * es);
    w.o = take(BH * d->T * d->d_v * es);
    w.gemm = take(kGemmWs);
    const kdn_desc c = core_desc(d);
    w.core = take(kdn_forward_workspace_bytes(&c));
    w.total = off;
    return w;
}

kdn_status check_layer(const kdn_layer_desc* d) {
    if (!d) return KDN_ERR_NULL;
    if (d->B < 0 || d->T < 0 || d->H < 0 || d->d_model < 0) return KDN_ERR_SHAPE;
    if (d->dtype != KDN_F32 && d->dtype != KDN_BF16) return KDN_ERR_UNSUPPORTED;
    // every row of the GEMM operands starts 16-byte aligned
    if (d->d_model % 8 != 0 || d->d_model == 0) return KDN_ERR_UNSUPPORTED;
    if (3 * d->H > 256) return KDN_ERR_UNSUPPORTED;  // gate threads of layer_in_kernel
    // token rows index grid.x and 32-bit GEMM sizes
    if (int64_t(d->B) * d->T > INT32_MAX) return KDN_ERR_UNSUPPORTED;
    if (int64_t(d->H) * (2 * d->d_k + d->d_v + 3) > INT32_MAX / 16) return KDN_ERR_UNSUPPORTED;
    const kdn_desc c = core_desc(d);
    return kdn_validate(&c);
}

char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The descriptors of one product (destroyed with the object)
struct GemmDescs {
    hipblasLtMatmulDesc_t op = nullptr;
    hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
    ~GemmDescs() {
        if (c) hipblasLtMatrixLayoutDestroy(c);
        if (b) hipblasLtMatrixLayoutDestroy(b);
        if (a) hipblasLtMatrixLayoutDestroy(a);
        if (op) hipblasLtMatmulDescDestroy(op);
    }
};

// row-major Y[M,N] = X[M,K] W^T, with W [N,K] row-major: in hipBLASLt's
// column-major terms Y^T (N x M, ld ldy) = op(A) B, A = W read as K x N (ld
// ldw) and transposed, B = X read as K x M (ld ldx): both operands contiguous
// along K.  The algorithm is hipBLASLt's first heuristic choice for the shape
// within kGemmWs of workspace, cached in the context.
template <typename E>
kdn_status gemm_rows(BlasCtx* bc, int M, int N, int K, const void* X, int ldx, const void* W,
                     int ldw, void* Y, int ldy, void* gws, hipStream_t st) {
    const hipDataType ty = Io<E>::blas;
    GemmDescs g;
    const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    if (hipblasLtMatmulDescCreate(&g.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatmulDescSetAttribute(g.op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) !=
            HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&g.a, ty, K, N, ldw) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&g.b, ty, K, M, ldx) != HIPBLAS_STATUS_SUCCESS ||
        hipblasLtMatrixLayoutCreate(&g.c, ty, N, M, ldy) != HIPBLAS_STATUS_SUCCESS)
        return KDN_ERR_HIP;
    hipblasLtMatmulAlgo_t algo;
    {
        std::lock_guard<std::mutex> lock(bc->mu);
        int found = -1;
        for (int i = 0; i < bc->n; ++i) {
            const BlasCtx::Entry& e = bc->cache[i];
            if (e.M == M && e.N == N && e.K == K && e.ldx == ldx && e.ldw == ldw &&
                e.ldy == ldy && e.type == ty) {
                found = i;
                break;
            }
        }
        if (found >= 0) {
            algo = bc->cache[found].algo;
        } else {
            hipblasLtMatmulPreference_t pref = nullptr;
            if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS)
                return KDN_ERR_HIP;
            const uint64_t cap = kGemmWs;
            hipblasLtMatmulHeuristicResult_t res[1];
            int got = 0;
            const bool ok =
                hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES,
                                                      &cap, sizeof(cap)) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatmulAlgoGetHeuristic(bc->lt, g.op, g.a, g.b, g.c, g.c, pref, 1, res,
                                                &got) == HIPBLAS_STATUS_SUCCESS &&
                got > 0 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize <= cap;
            hipblasLtMatmulPreferenceDestroy(pref);
            if (!ok) return KDN_ERR_HIP;
            algo = res[0].algo;
            const int slot = bc->n < 16 ? bc->n++ : 15;  // (a layer uses three shapes)
            bc->cache[slot] = {M, N, K, ldx, ldw, ldy, ty, algo};
        }
    }
    const float one = 1.f, zero = 0.f;
    return hipblasLtMatmul(bc->lt, g.op, &one, W, g.a, X, g.b, &zero, Y, g.c, Y, g.c, &algo, gws,
                           kGemmWs, st) == HIPBLAS_STATUS_SUCCESS
               ? KDN_OK
               : KDN_ERR_HIP;
}

// The same product with the output columns split at the last multiple of 128:
// the aligned block and the ragged rest as two products (at the layer shape
// the 48 gate columns after the 6,144 q, k, v columns).  W's rows are the
// output columns, so the second product starts N1 rows into W.
template <typename E>
kdn_status gemm_rows_split(BlasCtx* bc, int M, int N, int K, const void* X, int ldx,
                           const void* W, int ldw, void* Y, int ldy, void* gws, hipStream_t st) {
    const int N1 = N / 128 * 128;
    if (N1 == 0 || N1 == N) return gemm_rows<E>(bc, M, N, K, X, ldx, W, ldw, Y, ldy, gws, st);
    const kdn_status s = gemm_rows<E>(bc, M, N1, K, X, ldx, W, ldw, Y, ldy, gws, st);
    if (s != KDN_OK) return s;
    return gemm_rows<E>(bc, M, N - N1, K, X, ldx, static_cast<const E*>(W) + size_t(N1) * ldw,
                        ldw, static_cast<E*>(Y) + N1, ldy, gws, st);
}

template <typename E>
kdn_status layer_forward_t(const kdn_layer_desc* d, BlasCtx* hb, const void* x,
                           const void* W_in, const float* b_gate, const void* W_out,
                           const float* lambda0, const float* S0, void* y, float* S_T,
                           float* lambda_T, void* ws, const LayerWs& w, hipStream_t st,
                           void* const* events) {
    const int M = d->B * d->T, H = d->H, D = d->d_model, dk = d->d_k, dv = d->d_v;
    auto mark = [&](int i) -> bool {
        return !events || !events[i] ||
               hipEventRecord(static_cast<hipEvent_t>(events[i]), st) == hipSuccess;
    };
    void* Z = at(ws, w.z);
    void* gws = at(ws, w.gemm);
    void *q = at(ws, w.q), *k = at(ws, w.k), *v = at(ws, w.v);
    void *a = at(ws, w.a), *nu = at(ws, w.nu), *r = at(ws, w.r), *o = at(ws, w.o);
    if (!mark(0)) return KDN_ERR_HIP;
    kdn_status s = gemm_rows_split<E>(hb, M, n_in(d), D, x, D, W_in, D, Z, w.ldz, gws, st);
    if (s != KDN_OK || !mark(1) || !mark(2)) return s != KDN_OK ? s : KDN_ERR_HIP;
    if (launch_in<E>(dk, dv, Z, w.ldz, b_gate, M, H, d->T, q, k, v, a, nu, r, st) != hipSuccess)
        return KDN_ERR_HIP;
    if (!mark(3) || !mark(4)) return KDN_ERR_HIP;
    const kdn_desc c = core_desc(d);
    s = kdn_forward(&c, q, k, v, a, nu, r, lambda0, S0, o, S_T, lambda_T, at(ws, w.core),
                    w.total - w.core, st);
    if (s != KDN_OK) return s;
    if (!mark(5) || !mark(6)) return KDN_ERR_HIP;
    if (launch_out<E>(dv, o, Z, M, H, d->T, st) != hipSuccess) return KDN_ERR_HIP;
    if (!mark(7) || !mark(8)) return KDN_ERR_HIP;
    s = gemm_rows<E>(hb, M, D, H * dv, Z, H * dv, W_out, H * dv, y, D, gws, st);
    if (s != KDN_OK || !mark(9)) return s != KDN_OK ? s : KDN_ERR_HIP;
    return KDN_OK;
}

}  // namespace

extern "C" {

kdn_status kdn_blas_create(void** handle) {
    if (!handle) return KDN_ERR_NULL;
    BlasCtx* bc = new (std::nothrow) BlasCtx;
    if (!bc) return KDN_ERR_HIP;
    if (hipblasLtCreate(&bc->lt) != HIPBLAS_STATUS_SUCCESS) {
        delete bc;
        return KDN_ERR_HIP;
    }
    *handle = bc;
    return KDN_OK;
}

kdn_status kdn_blas_destroy(void* handle) {
    if (!handle) return KDN_OK;
    BlasCtx* bc = static_cast<BlasCtx*>(handle);
    const bool ok = hipblasLtDestroy(bc->lt) == HIPBLAS_STATUS_SUCCESS;
    delete bc;
    return ok ? KDN_OK : KDN_ERR_HIP;
}

size_t kdn_layer_workspace_bytes(const kdn_layer_desc* d) {
    if (check_layer(d) != KDN_OK) return 0;
    return layer_ws(d).total;
}

kdn_status kdn_layer_forward_events(const kdn_layer_desc* d, void* blas, const void* x,
                                    const void* W_in, const float* b_gate, const void* W_out,
                                    const float* lambda0, const float* S0, void* y, float* S_T,
                                    float* lambda_T, void* ws, size_t ws_bytes, void* stream,
                                    void* const* events) {
    kdn_status st = check_layer(d);
    if (st != KDN_OK) return st;
    if (size_t(d->B) * d->T == 0 || d->H == 0) {
        // no token rows: only the state passes through (the core call does that)
        const kdn_desc c = core_desc(d);
        if (d->B * d->H == 0) return KDN_OK;
        const LayerWs w = layer_ws(d);
        if (!ws) return KDN_ERR_NULL;
        if (ws_bytes < w.total) return KDN_ERR_WORKSPACE;
        return kdn_forward(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, lambda0, S0,
                           nullptr, S_T, lambda_T, at(ws, w.core), w.total - w.core, stream);
    }
    if (!blas || !x || !W_in || !b_gate || !W_out || !y || !ws) return KDN_ERR_NULL;
    const LayerWs w = layer_ws(d);
    if (ws_bytes < w.total) return KDN_ERR_WORKSPACE;
    for (const void* p : {x, W_in, W_out, (const void*)y, (const void*)ws})
        if (!aligned16(p)) return KDN_ERR_ALIGN;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    BlasCtx* hb = static_cast<BlasCtx*>(blas);
    return d->dtype == KDN_BF16
               ? layer_forward_t<bf16_t>(d, hb, x, W_in, b_gate, W_out, lambda0, S0, y, S_T,
                                         lambda_T, ws, w, hs, events)
               : layer_forward_t<float>(d, hb, x, W_in, b_gate, W_out, lambda0, S0, y, S_T,
                                        lambda_T, ws, w, hs, events);
}

kdn_status kdn_layer_forward(const kdn_layer_desc* d, void* blas, const void* x, const void* W_in,
                             const float* b_gate, const void* W_out, const float* lambda0,
                             const float* S0, void* y, float* S_T, float* lambda_T, void* ws,
                             size_t ws_bytes, void* stream) {
    return kdn_layer_forward_events(d, blas, x, W_in, b_gate, W_out, lambda0, S0, y, S_T,
                                    lambda_T, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"
