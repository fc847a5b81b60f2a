// kdn_dense.hip -- the exact KDN gain: the dense Riccati recursion with one
// d_k x d_k covariance per head ("Kalman Delta Networks", English abstract:
// tracking the key-space posterior exactly needs a full covariance whose
// Riccati update depends on the state; the diagonal and isotropic variants are
// the two cheap replacements for it).  Per token:
//   P^- = a^2 P + nu I,   w = P^- k / (k^T P^- k + r),
//   P   = P^- - (P^- k)(P^- k)^T / (k^T P^- k + r).
// The memory write with these gains is the generalised delta rule of the other
// variants (kdn_chunk_delta).
//
// One workgroup of 256 threads per head, sequential over the tokens.  P lives
// in registers as a 16 x 16 grid of (d_k/16)^2 blocks, one per lane; the 16
// lanes of a DPP row (one row of blocks) sum their parts of P^- k with DPP
// moves, so that each lane needs the key and P^- k only at its own d_k/16 rows
// and columns.  k^T P^- k comes from the same lane partials, DPP sums and four
// wave partials in LDS (the token's one barrier, which waits for LDS traffic
// only); P^- k is shared through LDS for the rank-one update.
//
// P is kept as s * Ps with a running scale s: the prediction a^2 P + nu I
// becomes s <- a^2 s and nu / s added to the diagonal of Ps, so that it costs
// nothing per entry; the update P^- - (P^- k)(P^- k)^T / den becomes
// Ps - c u u^T with u = Ps^- k and c = s / den, and the gain is c u.  When s
// leaves [2^-32, 2^32] (or a is zero) it is folded into Ps.  The two
// reciprocals per token are v_rcp_f32 (about 1 ulp), off the division's longer
// instruction sequence on the token's critical path.
//
// Keys and gates arrive in blocks of NB tokens: the next block is loaded into
// registers while the current one is worked on and moved into the other LDS
// buffer at its end, so that no token waits for global memory; the gains of a
// block collect in LDS and leave in 16-byte stores.  Per-token LDS buffers
// alternate between tokens, so that one barrier per token orders every access.
#include "kdn_device.h"
#include "kdn_launch.h"

namespace kdn {
namespace {

constexpr int kDenseNB = 32;  // tokens per staged block (even)

template <typename E> struct Vec16;  // 16 bytes of E
template <> struct Vec16<float> {
    using T = floatx4;
    static constexpr int N = 4;
    __device__ static void to_f(const T& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = v[i];
    }
    __device__ static T from_f(const float* f) { return T{f[0], f[1], f[2], f[3]}; }
};
template <> struct Vec16<bf16_t> {
    using T = u32x4;
    static constexpr int N = 8;
    __device__ static void to_f(const T& v, float* f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(v[i] << 16);
            f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
    }
    __device__ static T from_f(const float* f) {
        uint32_t u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = uint32_t(f2bf(f[2 * i])) | (uint32_t(f2bf(f[2 * i + 1])) << 16);
        return T{u[0], u[1], u[2], u[3]};
    }
};

template <typename E, typename G, int DK>
__global__ __launch_bounds__(256) void dense_gain_kernel(
    const E* __restrict__ k, const G* __restrict__ a, const G* __restrict__ nu,
    const G* __restrict__ r, const float* __restrict__ P0, E* __restrict__ w,
    float* __restrict__ P_T, int T) {
    constexpr int NB = kDenseNB;
    constexpr int BS = DK / 16;  // block edge: lane holds P[BS*rb + i][BS*cb + j]
    using V = Vec16<E>;
    constexpr int NV = NB * DK / V::N;              // 16-byte vectors of keys per block
    constexpr int VPT = (NV + 255) / 256;           // per thread
    __shared__ float kb[2][NB * DK], wb[2][NB * DK], gb[2][3][NB];
    __shared__ float us[2][DK], denp[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int rb = tid >> 4, cb = tid & 15;
    const bool lead = cb == 0, diag = rb == cb;
    const size_t bh = blockIdx.x, tok0 = bh * T;
    const typename V::T* kv = reinterpret_cast<const typename V::T*>(k + tok0 * DK);
    typename V::T* wv = reinterpret_cast<typename V::T*>(w + tok0 * DK);
    float P[BS][BS], sc = 1.f;  // P = sc * Ps
#pragma unroll
    for (int i = 0; i < BS; ++i)
#pragma unroll
        for (int j = 0; j < BS; ++j)
            P[i][j] = P0 ? P0[(bh * DK + BS * rb + i) * DK + BS * cb + j]
                         : (diag && i == j ? 1.f : 0.f);

    // registers holding the block being fetched
    typename V::T kpre[VPT];
    G gr = G(0);
#define KDN_DENSE_FETCH(base_)                                                          \
    {                                                                                  \
        const int nv_ = min(NB, T - (base_)) * (DK / V::N);                            \
        _Pragma("unroll") for (int i = 0; i < VPT; ++i) {                              \
            const int v = tid + 256 * i;                                               \
            if (v < nv_) kpre[i] = kv[size_t(base_) * (DK / V::N) + v];                \
        }                                                                              \
        if (tid < 3 * NB) {                                                            \
            const int g = tid / NB, t = (base_) + tid % NB;                            \
            const G* src = g == 0 ? a : g == 1 ? nu : r;                               \
            gr = t < T ? src[tok0 + t] : G(0);                                         \
        }                                                                              \
    }
#define KDN_DENSE_STAGE(buf_, base_)                                                    \
    {                                                                                  \
        const int nv_ = min(NB, T - (base_)) * (DK / V::N);                            \
        _Pragma("unroll") for (int i = 0; i < VPT; ++i) {                              \
            const int v = tid + 256 * i;                                               \
            if (v < nv_) V::to_f(kpre[i], &kb[buf_][v * V::N]);                        \
        }                                                                              \
        if (tid < 3 * NB) gb[buf_][tid / NB][tid % NB] = to_f<G>(gr);                  \
    }

    const int nblk = (T + NB - 1) / NB;
    if (nblk > 0) {
        KDN_DENSE_FETCH(0)
        KDN_DENSE_STAGE(0, 0)
    }
    // every load so far (P0 and the first block) complete before the token loop,
    // so that the compiler places no wait on them inside it
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int jb = 0; jb < nblk; ++jb) {
        const int buf = jb & 1, base = jb * NB, nt = min(NB, T - base);
        if (jb + 1 < nblk) KDN_DENSE_FETCH(base + NB)
        const float* kk = kb[buf];
        for (int tt = 0; tt < nt; ++tt) {
            const int b = tt & 1;
            const float* kt = kk + tt * DK;
            // predict: sc <- a^2 sc, nu / sc onto the diagonal of Ps
            const float at = gb[buf][0][tt], nut = gb[buf][1][tt];
            const float sn = sc * (at * at);
            if (!(sn >= 0x1p-32f && sn <= 0x1p32f)) {  // uniform: fold the scale into Ps
#pragma unroll
                for (int i = 0; i < BS; ++i)
#pragma unroll
                    for (int j = 0; j < BS; ++j) P[i][j] *= sn;
                sc = 1.f;
            } else {
                sc = sn;
            }
            if (diag) {
                const float add = nut * rcp(sc);
#pragma unroll
                for (int i = 0; i < BS; ++i) P[i][i] += add;
            }
            // u = Ps^- k at this lane's rows, from its columns; kr . u for k^T Ps^- k
            float kc[BS], kr[BS], u[BS];
#pragma unroll
            for (int j = 0; j < BS; ++j) {
                kc[j] = kt[BS * cb + j];
                kr[j] = kt[BS * rb + j];
            }
            float dp = 0.f;
#pragma unroll
            for (int i = 0; i < BS; ++i) {
                float x = 0.f;
#pragma unroll
                for (int j = 0; j < BS; ++j) x = fmaf(P[i][j], kc[j], x);
                u[i] = x;
                dp = fmaf(kr[i], x, dp);
            }
#pragma unroll
            for (int i = 0; i < BS; ++i) u[i] = group_sum<16>(u[i]);
            dp = group_sum<16>(dp);
            const float dw = lane_value(dp, 0) + lane_value(dp, 16) + lane_value(dp, 32) +
                             lane_value(dp, 48);
            if (lead) {
#pragma unroll
                for (int i = 0; i < BS; ++i) us[b][BS * rb + i] = u[i];
            }
            if (lane == 0) denp[b][wave] = dw;
            sync_lds();
            const float rt = gb[buf][2][tt];
            const float c =
                sc * rcp(rt + sc * (denp[b][0] + denp[b][1] + denp[b][2] + denp[b][3]));
            // rank-one update of Ps and the gain rows c u
            float ucol[BS];
#pragma unroll
            for (int j = 0; j < BS; ++j) ucol[j] = us[b][BS * cb + j];
#pragma unroll
            for (int i = 0; i < BS; ++i) {
                const float ci = c * u[i];
#pragma unroll
                for (int j = 0; j < BS; ++j) P[i][j] = fmaf(-ci, ucol[j], P[i][j]);
                if (lead) wb[buf][tt * DK + BS * rb + i] = ci;
            }
        }
        // the next block into the other buffers; this block's gains out
        if (jb + 1 < nblk) KDN_DENSE_STAGE(buf ^ 1, base + NB)
        sync_lds();
        const int nv = nt * (DK / V::N);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = tid + 256 * i;
            if (v < nv) wv[size_t(base) * (DK / V::N) + v] = V::from_f(&wb[buf][v * V::N]);
        }
    }
    if (P_T) {
#pragma unroll
        for (int i = 0; i < BS; ++i)
#pragma unroll
            for (int j = 0; j < BS; ++j)
                P_T[(bh * DK + BS * rb + i) * DK + BS * cb + j] = sc * P[i][j];
    }
#undef KDN_DENSE_FETCH
#undef KDN_DENSE_STAGE
}

template <typename E, typename G, int DK>
hipError_t dense_t(const Shape& s, const void* k, const void* a, const void* nu, const void* r,
                   const float* P0, void* w, float* P_T, hipStream_t st) {
    launch_k((dense_gain_kernel<E, G, DK>), dim3(s.BH), dim3(256), 0, st,
             static_cast<const E*>(k), static_cast<const G*>(a), static_cast<const G*>(nu),
             static_cast<const G*>(r), P0, static_cast<E*>(w), P_T, s.T);
    return hipGetLastError();
}

template <typename E>
hipError_t dense_e(const Shape& s, const void* k, const void* a, const void* nu, const void* r,
                   const float* P0, void* w, float* P_T, hipStream_t st) {
#define KDN_DENSE(DK_)                                                                   \
    if (s.dk == DK_)                                                                     \
        return s.gate_bf16 ? dense_t<E, bf16_t, DK_>(s, k, a, nu, r, P0, w, P_T, st)     \
                           : dense_t<E, float, DK_>(s, k, a, nu, r, P0, w, P_T, st);
    KDN_DENSE(32) KDN_DENSE(64) KDN_DENSE(128)
#undef KDN_DENSE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_dense_gain(const Shape& s, const void* k, const void* a, const void* nu,
                             const void* r, const float* P0, void* w, float* P_T,
                             hipStream_t st) {
    if (s.BH == 0) return hipSuccess;
    return s.qkv_bf16 ? dense_e<bf16_t>(s, k, a, nu, r, P0, w, P_T, st)
                      : dense_e<float>(s, k, a, nu, r, P0, w, P_T, st);
}

}  // namespace kdn
