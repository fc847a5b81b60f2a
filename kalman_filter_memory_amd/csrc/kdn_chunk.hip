// kdn_chunk.hip -- chunkwise memory write and read-out of the KDN layer.
//
// The memory recurrence S_t = a_t S_{t-1} + (v_t - a_t S_{t-1} k_t) w_t^T,
// o_t = S_t q_t is a generalised delta rule whose write key w_t is the Kalman
// gain ("Kalman Delta Networks", English abstract: the Kalman gain weights
// each residual write; ai-feeds.com summary, section 方法 step 3: hardware-
// efficient chunkwise implementation).  Within a chunk of C tokens that
// starts from S0, with local cumulative decay gamma_t = prod_{s<=t} a_s,
// g = log gamma and Gamma_ts = exp(g_t - g_s):
//   A  = strict_tril(K W^T * Gamma),  T = (I + A)^{-1}
//   U  = T (V - diag(gamma) K S0^T)                     (the innovations)
//   O  = diag(gamma) Q S0^T + (tril(Q W^T) * Gamma) U   (diagonal included)
//   S_end = gamma_C S0 + U^T diag(gamma_C / gamma_s) W
// Everything except the S0 terms is local to the chunk.
//
// Two kernels:
//   prep_kernel   one workgroup per chunk, all chunks in parallel: optionally
//                 the gain w from the chunk-boundary precision, then A and the
//                 unit-lower-triangular inverse T (16x16 diagonal blocks by
//                 forward substitution, off-diagonal blocks by block rows),
//                 all in fp32; T is stored in the input dtype.
//   state_kernel  one workgroup per (head, d_v tile), sequential over chunks:
//                 the S0-dependent products on MFMA (bf16 inputs: 16x16x32
//                 bf16 MFMA with fp32 accumulation; fp32 inputs: 16x16x4 fp32
//                 MFMA).  The fp32 state lives in MFMA accumulators for the
//                 whole sequence; an input-dtype copy of it is kept in LDS as
//                 the operand of the next chunk.
// Operand arrays in LDS are row-major with the contraction index contiguous,
// so every MFMA fragment is one 16-byte (bf16) or 4-byte (fp32) LDS read; the
// transposed copy of W needed by the state update is written when staged.
#include "kdn_device.h"
#include "kdn_kernels.h"

namespace kdn {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsLimit = 160 * 1024;

// ---------------------------------------------------------------- helpers
template <typename E> struct Vec16 {
    static constexpr int N = 16 / sizeof(E);
};

template <typename E>
__device__ __forceinline__ void store4(E* p, float x0, float x1, float x2, float x3);
template <>
__device__ __forceinline__ void store4<float>(float* p, float x0, float x1, float x2, float x3) {
    *reinterpret_cast<float4*>(p) = make_float4(x0, x1, x2, x3);
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float x0, float x1, float x2,
                                               float x3) {
    uint2 u;
    u.x = static_cast<uint32_t>(f2bf(x0)) | (static_cast<uint32_t>(f2bf(x1)) << 16);
    u.y = static_cast<uint32_t>(f2bf(x2)) | (static_cast<uint32_t>(f2bf(x3)) << 16);
    *reinterpret_cast<uint2*>(p) = u;
}

// inclusive prefix sum over the 64 lanes of a wave
__device__ __forceinline__ float wave_incl_sum(float x) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// copy `rows` x `cols` (cols * sizeof(E) a multiple of 16) from global rows of
// stride `gld` into LDS rows of stride `sld`; rows >= n are zero-filled
template <typename E, int ROWS, int COLS>
__device__ __forceinline__ void stage_rows(E* dst, int sld, const E* src, size_t gld, int n) {
    constexpr int V = Vec16<E>::N, VPR = COLS / V;
    for (int e = threadIdx.x; e < ROWS * VPR; e += kThreads) {
        const int t = e / VPR, c = (e % VPR) * V;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (t < n) val = *reinterpret_cast<const uint4*>(src + t * gld + c);
        *reinterpret_cast<uint4*>(dst + t * sld + c) = val;
    }
}

template <typename E, int DK, int C> struct PrepLds {
    static constexpr int PAD = Vec16<E>::N;
    static constexpr int LDK = DK + PAD, LDA = C + 1;
    static constexpr int NT = C / 16;
    static constexpr int FSZ = (C * DK > 2 * C * LDA) ? C * DK : 2 * C * LDA;
    static constexpr int ZSZ = (NT > 1 ? NT - 1 : 1) * 256;
    static constexpr int BYTES =
        2 * C * LDK * (int)sizeof(E) + (FSZ + 5 * C + ZSZ) * (int)sizeof(float);
};

template <typename E, int DK, int DVT, int C> struct StateLds {
    static constexpr int PAD = Vec16<E>::N;
    static constexpr int LDK = DK + PAD, LDC = C + PAD, LDV = DVT + PAD;
    static constexpr int BYTES =
        (3 * C * LDK + DK * LDC + DVT * LDK + DVT * LDC + 2 * C * LDC + C * LDV) *
            (int)sizeof(E) +
        C * (int)sizeof(float);
};

// ------------------------------------------------------------ prep kernel
template <typename E, int DK, int C>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const E* __restrict__ k, const void* __restrict__ a, const void* __restrict__ nu,
    const void* __restrict__ r, bool gate_bf16, bool diag, bool fuse_gain,
    const float* __restrict__ lam_chunk, E* __restrict__ w, E* __restrict__ Tm, int T, int NC) {
    using L = PrepLds<E, DK, C>;
    constexpr int LDK = L::LDK, LDA = L::LDA, NT = L::NT;
    constexpr int V = Vec16<E>::N, VPR = DK / V;
    __shared__ __align__(16) E sK[C * LDK];
    __shared__ __align__(16) E sW[C * LDK];
    __shared__ __align__(16) float sF[L::FSZ];  // lambda^- [C][DK], later A and T
    __shared__ float sa[C], snu[C], sr[C], sg[C], sden[C];
    __shared__ float sZ[L::ZSZ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = blockIdx.y;
    const int c = blockIdx.x;
    const int t0 = c * C, n = min(C, T - t0);
    const size_t row0 = bh * T + t0;

    stage_rows<E, C, DK>(sK, LDK, k + row0 * DK, DK, n);
    if (!fuse_gain) stage_rows<E, C, DK>(sW, LDK, w + row0 * DK, DK, n);
    if (tid < C) {
        const bool in = tid < n;  // padded tokens: a = 1, nu = 0, k = 0 (no effect)
        sa[tid] = in ? load_gate(a, row0 + tid, gate_bf16) : 1.f;
        snu[tid] = (in && fuse_gain) ? load_gate(nu, row0 + tid, gate_bf16) : 0.f;
        sr[tid] = (in && fuse_gain) ? load_gate(r, row0 + tid, gate_bf16) : 1.f;
    }
    __syncthreads();

    if (fuse_gain) {
        if (diag) {
            // predictive precision of every (token, key dim), sequential in t
            if (tid < DK) {
                float lam = lam_chunk[(bh * (NC + 1) + c) * DK + tid];
                for (int t = 0; t < C; ++t) {
                    const float at = sa[t];
                    const float lm = lam / (at * at + snu[t] * lam);
                    sF[t * DK + tid] = lm;
                    const float kv = to_f<E>(sK[t * LDK + tid]);
                    lam = lm + kv * kv / sr[t];
                }
            }
            __syncthreads();
            if (tid < C) {  // gain denominator k^T P^- k + r per token
                float den = sr[tid];
                for (int i = 0; i < DK; ++i) {
                    const float kv = to_f<E>(sK[tid * LDK + i]);
                    den += kv * kv / sF[tid * DK + i];
                }
                sden[tid] = 1.f / den;
            }
        } else {
            if (tid < C) {
                float kk = 0.f;
                for (int i = 0; i < DK; ++i) {
                    const float kv = to_f<E>(sK[tid * LDK + i]);
                    kk += kv * kv;
                }
                sden[tid] = kk;
            }
            __syncthreads();
            if (tid == 0) {  // one precision per head: w = k / (|k|^2 + r lambda^-)
                float lam = lam_chunk[bh * (NC + 1) + c];
                for (int t = 0; t < C; ++t) {
                    const float at = sa[t], kk = sden[t];
                    const float lm = lam / (at * at + snu[t] * lam);
                    sden[t] = 1.f / (kk + sr[t] * lm);
                    lam = lm + kk / (static_cast<float>(DK) * sr[t]);
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < C * VPR; e += kThreads) {
            const int t = e / VPR, i0 = (e % VPR) * V;
            E out[V];
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const float kv = to_f<E>(sK[t * LDK + i0 + j]);
                const float pk = diag ? kv / sF[t * DK + i0 + j] : kv;
                out[j] = from_f<E>(pk * sden[t]);
            }
            const uint4 u = *reinterpret_cast<const uint4*>(out);
            *reinterpret_cast<uint4*>(sW + t * LDK + i0) = u;
            if (t < n) *reinterpret_cast<uint4*>(w + (row0 + t) * DK + i0) = u;
        }
    }
    if (wave == 0) {
        const float la = wave_incl_sum(lane < C ? logf(sa[lane]) : 0.f);
        if (lane < C) sg[lane] = la;
    }
    __syncthreads();

    // A = strict_tril(K W^T * Gamma) in fp32; T zero-initialised
    float* sA = sF;
    float* sT = sF + C * LDA;
    for (int id = wave; id < NT * NT; id += 4) {
        const int tb = id / NT, sb = id % NT;
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        if (sb <= tb) acc = mma_tile<E>(acc, sK, LDK, 16 * tb, sW, LDK, 16 * sb, 0, DK, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * tb + c_row(lane, e), s = 16 * sb + c_col(lane);
            sA[t * LDA + s] = (s < t) ? expf(sg[t] - sg[s]) * acc[e] : 0.f;
        }
    }
    for (int e = tid; e < C * LDA; e += kThreads) sT[e] = 0.f;
    __syncthreads();

    // diagonal 16x16 blocks: forward substitution, one lane per column
    if (wave < NT && lane < 16) {
        const int b0 = 16 * wave;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float acc = (t == lane) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < t; ++s) acc -= sA[(b0 + t) * LDA + b0 + s] * x[s];
            x[t] = acc;
            sT[(b0 + t) * LDA + b0 + lane] = acc;
        }
    }
    __syncthreads();
    // block row i: T_ij = -T_ii * sum_{m=j}^{i-1} A_im T_mj
    for (int i = 1; i < NT; ++i) {
        for (int e = tid; e < i * 256; e += kThreads) {
            const int j = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            float acc = 0.f;
            for (int m = 16 * j; m < 16 * i; ++m)
                acc += sA[(16 * i + rr) * LDA + m] * sT[m * LDA + 16 * j + cc];
            sZ[e] = acc;
        }
        __syncthreads();
        for (int e = tid; e < i * 256; e += kThreads) {
            const int j = e >> 8, rr = (e >> 4) & 15, cc = e & 15;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m)
                acc += sT[(16 * i + rr) * LDA + 16 * i + m] * sZ[(j << 8) + (m << 4) + cc];
            sT[(16 * i + rr) * LDA + 16 * j + cc] = -acc;
        }
        __syncthreads();
    }
    E* Tout = Tm + (bh * NC + c) * (size_t)(C * C);
    for (int e = tid; e < C * C; e += kThreads) Tout[e] = from_f<E>(sT[(e / C) * LDA + e % C]);
}

// ----------------------------------------------------------- state kernel
template <typename E, int DK, int DVT, int C>
__global__ __launch_bounds__(kThreads) void state_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const void* __restrict__ a, bool gate_bf16, const E* __restrict__ w,
    const E* __restrict__ Tm, const float* S0, E* __restrict__ o, float* S_T, int T, int DV,
    int NC) {
    using L = StateLds<E, DK, DVT, C>;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDV = L::LDV;
    constexpr int NT = C / 16, NK = DK / 16, NV = DVT / 16;
    constexpr int NS = (NK * NV + 3) / 4;  // state tiles per wave
    constexpr int NO = (NV * NT + 3) / 4;  // output / innovation tiles per wave
    __shared__ __align__(16) E sK[C * LDK];
    __shared__ __align__(16) E sW[C * LDK];
    __shared__ __align__(16) E sQ[C * LDK];
    __shared__ __align__(16) E sWt[DK * LDC];  // (gamma_C / gamma_t) W, transposed [i][t]
    __shared__ __align__(16) E sS[DVT * LDK];  // S tile [j][i] as operand
    __shared__ __align__(16) E sRU[DVT * LDC]; // R^T, then U^T  [j][t]
    __shared__ __align__(16) E sT[C * LDC];    // (I + A)^{-1}    [t][s]
    __shared__ __align__(16) E sM[C * LDC];    // tril(Q W^T) * Gamma  [t][s]
    __shared__ __align__(16) E sV[C * LDV];
    __shared__ float sg[C];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = blockIdx.y;
    const int j0 = blockIdx.x * DVT;

    // state tile (bi, bj) of S^T: element e <-> i = 16 bi + 4 (lane/16) + e, j = 16 bj + lane%16
    floatx4 accS[NS];
#pragma unroll
    for (int x = 0; x < NS; ++x) {
        accS[x] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int id = wave + 4 * x;
        if (id < NK * NV && S0) {
            const int i = 16 * (id / NV) + 4 * (lane >> 4), j = 16 * (id % NV) + (lane & 15);
            const float4 s4 =
                *reinterpret_cast<const float4*>(S0 + (bh * DV + j0 + j) * DK + i);
            accS[x] = floatx4{s4.x, s4.y, s4.z, s4.w};
        }
    }
#pragma unroll
    for (int x = 0; x < NS; ++x) {
        const int id = wave + 4 * x;
        if (id < NK * NV) {
            const int i = 16 * (id / NV) + 4 * (lane >> 4), j = 16 * (id % NV) + (lane & 15);
            store4<E>(sS + j * LDK + i, accS[x][0], accS[x][1], accS[x][2], accS[x][3]);
        }
    }

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * C, n = min(C, T - t0);
        const size_t row0 = bh * T + t0;
        stage_rows<E, C, DK>(sK, LDK, k + row0 * DK, DK, n);
        stage_rows<E, C, DK>(sW, LDK, w + row0 * DK, DK, n);
        stage_rows<E, C, DK>(sQ, LDK, q + row0 * DK, DK, n);
        stage_rows<E, C, DVT>(sV, LDV, v + row0 * DV + j0, DV, n);
        stage_rows<E, C, C>(sT, LDC, Tm + (bh * NC + c) * (size_t)(C * C), C, C);
        if (wave == 0) {
            const float la = wave_incl_sum(
                lane < n ? logf(load_gate(a, row0 + lane, gate_bf16)) : 0.f);
            if (lane < C) sg[lane] = la;
        }
        __syncthreads();
        const float glast = sg[C - 1];

        // transposed, decay-weighted W for the state update
        {
            constexpr int V = Vec16<E>::N, VPR = DK / V;
            for (int e = tid; e < C * VPR; e += kThreads) {
                const int t = e / VPR, i0 = (e % VPR) * V;
                const float sc = expf(glast - sg[t]);
                E vals[V];
                *reinterpret_cast<uint4*>(vals) =
                    *reinterpret_cast<const uint4*>(sW + t * LDK + i0);
#pragma unroll
                for (int j = 0; j < V; ++j)
                    sWt[(i0 + j) * LDC + t] = from_f<E>(sc * to_f<E>(vals[j]));
            }
        }
        // M^T = W Q^T, stored as M[t][s] (zero where s > t)
        for (int id = wave; id < NT * NT; id += 4) {
            const int sb = id / NT, tb = id % NT;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
            if (sb <= tb) acc = mma_tile<E>(acc, sW, LDK, 16 * sb, sQ, LDK, 16 * tb, 0, DK, lane);
            const int t = 16 * tb + c_col(lane), s = 16 * sb + c_row(lane, 0);
            float m4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) m4[e] = (s + e <= t) ? expf(sg[t] - sg[s + e]) * acc[e] : 0.f;
            store4<E>(sM + t * LDC + s, m4[0], m4[1], m4[2], m4[3]);
        }
        // R = V - diag(gamma) K S^T  -> R^T;   O^T accumulators start at gamma_t (S Q^T)
        floatx4 accO[NO];
#pragma unroll
        for (int x = 0; x < NO; ++x) {
            accO[x] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int id = wave + 4 * x;
            if (id < NT * NV) {
                const int tb = id / NV, jb = id % NV;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_tile<E>(acc, sK, LDK, 16 * tb, sS, LDK, 16 * jb, 0, DK, lane);
                const int t = 16 * tb + c_row(lane, 0), j = 16 * jb + c_col(lane);
                float r4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r4[e] = to_f<E>(sV[(t + e) * LDV + j]) - expf(sg[t + e]) * acc[e];
                store4<E>(sRU + j * LDC + t, r4[0], r4[1], r4[2], r4[3]);
            }
            if (id < NV * NT) {
                const int jb = id / NT, tb = id % NT;
                floatx4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_tile<E>(acc, sS, LDK, 16 * jb, sQ, LDK, 16 * tb, 0, DK, lane);
                const float gt = expf(sg[16 * tb + c_col(lane)]);
                accO[x] = acc * gt;
            }
        }
        __syncthreads();

        // U = T R  (T lower triangular: contraction only up to the tile's last row)
        floatx4 accU[NO];
#pragma unroll
        for (int x = 0; x < NO; ++x) {
            accU[x] = floatx4{0.f, 0.f, 0.f, 0.f};
            const int id = wave + 4 * x;
            if (id < NT * NV) {
                const int tb = id / NV, jb = id % NV;
                const int kend = 16 * (tb + 1);
                accU[x] = mma_tile<E>(accU[x], sT, LDC, 16 * tb, sRU, LDC, 16 * jb, 0, kend, lane);
            }
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < NO; ++x) {
            const int id = wave + 4 * x;
            if (id < NT * NV) {
                const int tb = id / NV, jb = id % NV;
                const int t = 16 * tb + c_row(lane, 0), j = 16 * jb + c_col(lane);
                store4<E>(sRU + j * LDC + t, accU[x][0], accU[x][1], accU[x][2], accU[x][3]);
            }
        }
        __syncthreads();

        // O^T += U^T M^T  and write o
#pragma unroll
        for (int x = 0; x < NO; ++x) {
            const int id = wave + 4 * x;
            if (id < NV * NT) {
                const int jb = id / NT, tb = id % NT;
                const int kend = 16 * (tb + 1);
                accO[x] = mma_tile<E>(accO[x], sRU, LDC, 16 * jb, sM, LDC, 16 * tb, 0, kend, lane);
                const int t = 16 * tb + c_col(lane), j = 16 * jb + c_row(lane, 0);
                if (t < n)
                    store4<E>(o + (row0 + t) * DV + j0 + j, accO[x][0], accO[x][1], accO[x][2],
                              accO[x][3]);
            }
        }
        // S^T <- gamma_C S^T + Wbar^T U
        const float gC = expf(glast);
#pragma unroll
        for (int x = 0; x < NS; ++x) {
            const int id = wave + 4 * x;
            if (id < NK * NV) {
                const int bi = id / NV, bj = id % NV;
                accS[x] = accS[x] * gC;
                accS[x] = mma_tile<E>(accS[x], sWt, LDC, 16 * bi, sRU, LDC, 16 * bj, 0, C, lane);
            }
        }
        __syncthreads();
#pragma unroll
        for (int x = 0; x < NS; ++x) {
            const int id = wave + 4 * x;
            if (id < NK * NV) {
                const int i = 16 * (id / NV) + 4 * (lane >> 4), j = 16 * (id % NV) + (lane & 15);
                store4<E>(sS + j * LDK + i, accS[x][0], accS[x][1], accS[x][2], accS[x][3]);
            }
        }
    }
    if (S_T) {
#pragma unroll
        for (int x = 0; x < NS; ++x) {
            const int id = wave + 4 * x;
            if (id < NK * NV) {
                const int i = 16 * (id / NV) + 4 * (lane >> 4), j = 16 * (id % NV) + (lane & 15);
                *reinterpret_cast<float4*>(S_T + (bh * DV + j0 + j) * DK + i) =
                    make_float4(accS[x][0], accS[x][1], accS[x][2], accS[x][3]);
            }
        }
    }
}

// ---------------------------------------------------------------- dispatch
int dv_tile(int dv) { return dv < 64 ? dv : 64; }

template <typename E, int DK, int C>
hipError_t prep_t(const Shape& s, bool fuse, const void* k, const void* a, const void* nu,
                  const void* r, const float* lc, void* w, void* Tm, hipStream_t st) {
    static_assert(PrepLds<E, DK, C>::BYTES <= kLdsLimit, "prep LDS");
    hipLaunchKernelGGL((prep_kernel<E, DK, C>), dim3(s.nc, s.BH), dim3(kThreads), 0, st,
                       static_cast<const E*>(k), a, nu, r, s.gate_bf16, s.diag, fuse, lc,
                       static_cast<E*>(w), static_cast<E*>(Tm), s.T, s.nc);
    return hipGetLastError();
}

template <typename E, int DK, int DVT, int C>
hipError_t state_t(const Shape& s, const void* q, const void* k, const void* v, const void* a,
                   const void* w, const void* Tm, const float* S0, void* o, float* S_T,
                   hipStream_t st) {
    if constexpr (StateLds<E, DK, DVT, C>::BYTES <= kLdsLimit) {
        hipLaunchKernelGGL((state_kernel<E, DK, DVT, C>), dim3(s.dv / DVT, s.BH),
                           dim3(kThreads), 0, st, static_cast<const E*>(q),
                           static_cast<const E*>(k), static_cast<const E*>(v), a, s.gate_bf16,
                           static_cast<const E*>(w), static_cast<const E*>(Tm), S0,
                           static_cast<E*>(o), S_T, s.T, s.dv, s.nc);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <typename E, int DK, int DVT, int C>
constexpr bool state_fits() {
    return StateLds<E, DK, DVT, C>::BYTES <= kLdsLimit;
}

template <typename E>
bool supported_e(int dk, int dvt, int C) {
#define KDN_SUP(DK_, DVT_, C_) \
    if (dk == DK_ && dvt == DVT_ && C == C_) return state_fits<E, DK_, DVT_, C_>();
#define KDN_SUP_C(DK_, DVT_) KDN_SUP(DK_, DVT_, 16) KDN_SUP(DK_, DVT_, 32) KDN_SUP(DK_, DVT_, 64)
    KDN_SUP_C(32, 32) KDN_SUP_C(32, 64) KDN_SUP_C(64, 32) KDN_SUP_C(64, 64)
    KDN_SUP_C(128, 32) KDN_SUP_C(128, 64)
#undef KDN_SUP_C
#undef KDN_SUP
    return false;
}

template <typename E>
hipError_t prep_e(const Shape& s, bool fuse, const void* k, const void* a, const void* nu,
                  const void* r, const float* lc, void* w, void* Tm, hipStream_t st) {
#define KDN_PREP(DK_, C_) \
    if (s.dk == DK_ && s.chunk == C_) return prep_t<E, DK_, C_>(s, fuse, k, a, nu, r, lc, w, Tm, st);
#define KDN_PREP_C(DK_) KDN_PREP(DK_, 16) KDN_PREP(DK_, 32) KDN_PREP(DK_, 64)
    KDN_PREP_C(32) KDN_PREP_C(64) KDN_PREP_C(128)
#undef KDN_PREP_C
#undef KDN_PREP
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t state_e(const Shape& s, const void* q, const void* k, const void* v, const void* a,
                   const void* w, const void* Tm, const float* S0, void* o, float* S_T,
                   hipStream_t st) {
    const int dvt = dv_tile(s.dv);
#define KDN_ST(DK_, DVT_, C_)                                                             \
    if (s.dk == DK_ && dvt == DVT_ && s.chunk == C_)                                      \
        return state_t<E, DK_, DVT_, C_>(s, q, k, v, a, w, Tm, S0, o, S_T, st);
#define KDN_ST_C(DK_, DVT_) KDN_ST(DK_, DVT_, 16) KDN_ST(DK_, DVT_, 32) KDN_ST(DK_, DVT_, 64)
    KDN_ST_C(32, 32) KDN_ST_C(32, 64) KDN_ST_C(64, 32) KDN_ST_C(64, 64)
    KDN_ST_C(128, 32) KDN_ST_C(128, 64)
#undef KDN_ST_C
#undef KDN_ST
    return hipErrorInvalidValue;
}

}  // namespace

bool chunk_supported(const Shape& s) {
    auto ok = [](int d) { return d == 32 || d == 64 || d == 128; };
    if (!ok(s.dk) || !ok(s.dv)) return false;
    if (s.chunk != 16 && s.chunk != 32 && s.chunk != 64) return false;
    return s.qkv_bf16 ? supported_e<bf16_t>(s.dk, dv_tile(s.dv), s.chunk)
                      : supported_e<float>(s.dk, dv_tile(s.dv), s.chunk);
}

hipError_t launch_chunk_prep(const Shape& s, bool fuse_gain, const void* k, const void* a,
                             const void* nu, const void* r, const float* lam_chunk, void* w,
                             void* Tm, hipStream_t st) {
    if (s.BH == 0 || s.nc == 0) return hipSuccess;
    return s.qkv_bf16 ? prep_e<bf16_t>(s, fuse_gain, k, a, nu, r, lam_chunk, w, Tm, st)
                      : prep_e<float>(s, fuse_gain, k, a, nu, r, lam_chunk, w, Tm, st);
}

hipError_t launch_chunk_state(const Shape& s, const void* q, const void* k, const void* v,
                              const void* a, const void* w, const void* Tm, const float* S0,
                              void* o, float* S_T, hipStream_t st) {
    if (s.BH == 0) return hipSuccess;
    return s.qkv_bf16 ? state_e<bf16_t>(s, q, k, v, a, w, Tm, S0, o, S_T, st)
                      : state_e<float>(s, q, k, v, a, w, Tm, S0, o, S_T, st);
}

}  // namespace kdn
