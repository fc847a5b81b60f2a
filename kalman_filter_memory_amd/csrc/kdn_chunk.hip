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

template <typename E> __device__ __forceinline__ void load4(const E* p, float (&x)[4]);
template <> __device__ __forceinline__ void load4<float>(const float* p, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x;
    x[1] = v.y;
    x[2] = v.z;
    x[3] = v.w;
}
template <> __device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float (&x)[4]) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xFFFF0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xFFFF0000u);
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
    constexpr int V = Vec16<E>::N, VPR = COLS / V, NV = ROWS * VPR;
    constexpr int ITER = (NV + kThreads - 1) / kThreads;
    uint4 val[ITER];
#pragma unroll
    for (int x = 0; x < ITER; ++x) {  // all loads first (unconditional, clamped row)
        const int e = threadIdx.x + kThreads * x;
        const int t = e / VPR, c = (e % VPR) * V;
        if (e < NV) val[x] = *reinterpret_cast<const uint4*>(src + min(t, n - 1) * gld + c);
    }
#pragma unroll
    for (int x = 0; x < ITER; ++x) {
        const int e = threadIdx.x + kThreads * x;
        const int t = e / VPR, c = (e % VPR) * V;
        if (e < NV) {
            if (t >= n) val[x] = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(dst + t * sld + c) = val[x];
        }
    }
}

template <typename E, int DK, int C> struct PrepLds {
    static constexpr int PAD = Vec16<E>::N;
    static constexpr int LDK = DK + PAD, LDA = C + 4, LDP = DK + 4;
    static constexpr int NT = C / 16;
    static constexpr int FSZ = (C * LDP > 2 * C * LDA) ? C * LDP : 2 * C * LDA;
    static constexpr int ZSZ = (NT > 1 ? NT - 1 : 1) * 256;
    static constexpr int BYTES =
        2 * C * LDK * (int)sizeof(E) + (FSZ + 2 * C + ZSZ) * (int)sizeof(float);
};

// ------------------------------------------------------------ prep kernel
// One workgroup (4 waves) per chunk.
//   gain (fuse_gain): from the chunk-boundary precision, the predictive
//     precision of every (token, key dim) by the step recurrence (diagonal:
//     one lane per key dim, token scalars broadcast from the lane that loaded
//     them; isotropic: one scalar chain), P^- k into LDS, the per-token
//     denominator k^T P^- k + r (four lanes per token, a quarter of the key
//     dims each), then w = P^- k / (k^T P^- k + r).
//   A = strict_tril(K W^T * Gamma) on MFMA, T = (I + A)^{-1} in fp32:
//     16x16 diagonal blocks by forward substitution (one lane per column),
//     then block rows T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj with fp32 MFMA.
template <typename E, int DK, int C>
__global__ __launch_bounds__(kThreads) void prep_kernel(
    const E* __restrict__ k, const void* __restrict__ a, const void* __restrict__ nu,
    const void* __restrict__ r, bool gate_bf16, bool diag, bool fuse_gain,
    const float* __restrict__ lam_chunk, E* __restrict__ w, E* __restrict__ Tm, int T, int NC) {
    using L = PrepLds<E, DK, C>;
    constexpr int LDK = L::LDK, LDA = L::LDA, LDP = L::LDP, NT = L::NT;
    constexpr int V = Vec16<E>::N, VPR = DK / V;
    __shared__ __align__(16) E sK[C * LDK];
    __shared__ __align__(16) E sW[C * LDK];
    __shared__ __align__(16) float sF[L::FSZ];  // P^- k [C][LDP], later A and T [C][LDA]
    __shared__ __align__(16) float sden[C];
    __shared__ __align__(16) float sg[C];
    __shared__ __align__(16) float sZ[L::ZSZ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = blockIdx.y;
    const int c = blockIdx.x;
    const int t0 = c * C, n = min(C, T - t0);
    const size_t row0 = bh * T + t0;

    stage_rows<E, C, DK>(sK, LDK, k + row0 * DK, DK, n);
    if (!fuse_gain) stage_rows<E, C, DK>(sW, LDK, w + row0 * DK, DK, n);
    // lane t of every wave: the gates of token t (padding: a = 1, nu = 0, r = 1)
    float ga = 1.f, ga2 = 1.f, gnu = 0.f, gr = 1.f, gir = 1.f;
    {
        const size_t tok = row0 + min(lane, n - 1);
        const float at = load_gate(a, tok, gate_bf16);
        float rt = 1.f, nut = 0.f;
        if (fuse_gain) {
            rt = load_gate(r, tok, gate_bf16);
            nut = load_gate(nu, tok, gate_bf16);
        }
        if (lane < n) {
            ga = at;
            ga2 = at * at;
            gnu = nut;
            gr = rt;
            gir = 1.f / rt;
        }
    }
    sync_lds();

    if (fuse_gain) {
        if (diag) {
            // predictive precision, sequential in t, one lane per key dim;
            // stores P^- k = k (a^2 + nu lambda) / lambda
            if (tid < DK) {
                float lam = lam_chunk[(bh * (NC + 1) + c) * DK + tid];
#pragma unroll 8
                for (int t = 0; t < C; ++t) {
                    const float a2 = lane_value(ga2, t), nut = lane_value(gnu, t);
                    const float ir = lane_value(gir, t);
                    const float kv = to_f<E>(sK[t * LDK + tid]);
                    const float d = fmaf(nut, lam, a2);
                    sF[t * LDP + tid] = kv * d * rcp(lam);
                    const float lm = lam * rcp(d);
                    lam = fmaf(kv * kv, ir, lm);
                }
            }
            sync_lds();
            // denominators: four lanes per token, a quarter of the key dims each
            {
                constexpr int Q = DK / 4;
                const int t = wave * 16 + (lane >> 2), qd = lane & 3;
                float part = 0.f;
                if (t < C) {
#pragma unroll
                    for (int m = 0; m < Q; m += 4) {
                        const float4 pv = *reinterpret_cast<const float4*>(sF + t * LDP + qd * Q + m);
                        float kv[4];
                        load4<E>(sK + t * LDK + qd * Q + m, kv);
                        part += kv[0] * pv.x + kv[1] * pv.y + kv[2] * pv.z + kv[3] * pv.w;
                    }
                }
                part += __shfl_xor(part, 1, kWave);
                part += __shfl_xor(part, 2, kWave);
                if (t < C && qd == 0) sden[t] = part;
            }
            sync_lds();
            if (tid < C) sden[tid] = 1.f / (sden[tid] + gr);  // wave 0: lane t holds r_t
        } else {
            // |k|^2 per token, then one scalar chain: w = k / (|k|^2 + r lambda^-)
            {
                constexpr int Q = DK / 4;
                const int t = wave * 16 + (lane >> 2), qd = lane & 3;
                float part = 0.f;
                if (t < C) {
#pragma unroll
                    for (int m = 0; m < Q; m += 4) {
                        float kv[4];
                        load4<E>(sK + t * LDK + qd * Q + m, kv);
                        part += kv[0] * kv[0] + kv[1] * kv[1] + kv[2] * kv[2] + kv[3] * kv[3];
                    }
                }
                part += __shfl_xor(part, 1, kWave);
                part += __shfl_xor(part, 2, kWave);
                if (t < C && qd == 0) sden[t] = part;
            }
            sync_lds();
            if (wave == 0) {
                const float kk_l = lane < C ? sden[lane] : 0.f;
                float lam = lam_chunk[bh * (NC + 1) + c];
                float den_l = 1.f;
                for (int t = 0; t < C; ++t) {
                    const float kk = lane_value(kk_l, t);
                    const float lm = lam * rcp(fmaf(lane_value(gnu, t), lam, lane_value(ga2, t)));
                    if (lane == t) den_l = 1.f / (kk + lane_value(gr, t) * lm);
                    lam = fmaf(kk, lane_value(gir, t) * (1.f / static_cast<float>(DK)), lm);
                }
                if (lane < C) sden[lane] = den_l;
            }
        }
        sync_lds();
        for (int e = tid; e < C * VPR; e += kThreads) {
            const int t = e / VPR, i0 = (e % VPR) * V;
            E out[V];
            const float dn = sden[t];
#pragma unroll
            for (int j = 0; j < V; ++j) {
                const float pk = diag ? sF[t * LDP + i0 + j] : to_f<E>(sK[t * LDK + i0 + j]);
                out[j] = from_f<E>(pk * dn);
            }
            const uint4 u = *reinterpret_cast<const uint4*>(out);
            *reinterpret_cast<uint4*>(sW + t * LDK + i0) = u;
            if (t < n) *reinterpret_cast<uint4*>(w + (row0 + t) * DK + i0) = u;
        }
    }
    if (wave == 0) {
        const float g = wave_incl_sum(lane < C ? log2_hw(ga) : 0.f);
        if (lane < C) sg[lane] = g;
    }
    sync_lds();

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
            sA[t * LDA + s] = (s < t) ? exp2_hw(sg[t] - sg[s]) * acc[e] : 0.f;
        }
    }
    for (int e = tid; e < C * LDA; e += kThreads) sT[e] = 0.f;
    sync_lds();

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
    sync_lds();
    // block row i: Z_j = sum_{m=j}^{i-1} A_im T_mj, then T_ij = -T_ii Z_j
    // (16x16x16 products on fp32 MFMA; T is read k-major as the B operand)
    for (int i = 1; i < NT; ++i) {
        for (int j = wave; j < i; j += 4) {
            floatx4 z[1][1] = {{floatx4{0.f, 0.f, 0.f, 0.f}}};
            for (int m = j; m < i; ++m)
                mma_block<float, 1, 1, false, true>(z, sA + 16 * m, LDA, 16 * i,
                                                    sT + 16 * m * LDA, LDA, 16 * j, 0, 16, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sZ[(j << 8) + (c_row(lane, e) << 4) + c_col(lane)] = z[0][0][e];
        }
        sync_lds();
        for (int j = wave; j < i; j += 4) {
            floatx4 tij[1][1] = {{floatx4{0.f, 0.f, 0.f, 0.f}}};
            mma_block<float, 1, 1, false, true>(tij, sT + 16 * i, LDA, 16 * i, sZ + (j << 8), 16,
                                                0, 0, 16, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sT[(16 * i + c_row(lane, e)) * LDA + 16 * j + c_col(lane)] = -tij[0][0][e];
        }
        sync_lds();
    }
    E* Tout = Tm + (bh * NC + c) * (size_t)(C * C);
    for (int e = tid; e < C * C / V; e += kThreads) {
        const int t = e / (C / V), s0 = (e % (C / V)) * V;
        E out[V];
#pragma unroll
        for (int j = 0; j < V; ++j) out[j] = from_f<E>(sT[t * LDA + s0 + j]);
        *reinterpret_cast<uint4*>(Tout + t * C + s0) = *reinterpret_cast<const uint4*>(out);
    }
}

// ----------------------------------------------------------- state kernel
// One workgroup of 8 waves per (head, d_v tile), sequential over the chunks.
// Per chunk, with S the state at the chunk start and gamma_t = 2^(g_t):
//   phase A  every wave, one (2 j-tiles x 1 t-tile) block:
//              X^T = S K^T  ->  R = V - diag(gamma) X   (stored token-major)
//              Y   = diag(gamma) Q S^T, kept as the O^T accumulator
//            (both products share the S fragments)
//   phase B  waves 0-3: U = T R (stored as U^T, and as U^T scaled by
//            gamma_C / gamma_t); waves 4-7: M = tril(Q W^T) * Gamma
//   phase C  every wave: O^T += U^T M^T for its block, written out; and one
//            block of the state update S^T <- gamma_C S^T + W^T diag(gamma_C/gamma_t) U
//   phase D  the next chunk's K, W, Q, V, T, a (loaded from HBM into registers
//            at the start of this chunk) are written to LDS together with its
//            decay tables; the new state is written to LDS as the next operand.
// Operands stored with the contraction index strided (token-major R and W) are
// read with transposing LDS reads (ds_read_b64_tr_b16).  Barriers are LDS-only
// (sync_lds) so that the next chunk's global loads stay in flight across them.
// Decays use base-2 logarithms: g_t = sum_{s<=t} log2 a_s, Gamma_ts = 2^(g_t-g_s).
template <typename E, int DK, int DVT, int C> struct StateCfg {
    static constexpr int NW = 8, THREADS = 64 * NW;
    static constexpr int PAD = Vec16<E>::N, VEC = Vec16<E>::N;
    static constexpr int LDK = DK + PAD, LDC = C + PAD, LDV = DVT + PAD;
    static constexpr int NT = C / 16, NK = DK / 16, NV = DVT / 16;
    // phase A / O blocks: BVA j-tiles x 1 t-tile
    static constexpr int BVA = NV >= 2 ? 2 : 1;
    static constexpr int NAJ = (NV / BVA) * NT;
    static constexpr int APW = (NAJ + NW - 1) / NW;
    // phase B blocks: BT x BV tiles
    static constexpr int BT = NT >= 2 ? 2 : 1, BV = NV >= 2 ? 2 : 1, BI = 2;
    static constexpr int NTB = NT / BT, NVB = NV / BV, NIB = NK / BI;
    static constexpr int NUJ = NTB * NVB;            // U blocks (waves 0-3)
    static constexpr int NMJ = NTB * (NTB + 1) / 2;  // lower-triangular M blocks (waves 4-7)
    static constexpr int UPW = (NUJ + 3) / 4, MPW = (NMJ + 3) / 4;
    static constexpr int NSJ = NIB * NVB;            // state blocks
    static constexpr int SPW = (NSJ + NW - 1) / NW;
    static constexpr int NVK = C * DK / VEC, NVV = C * DVT / VEC, NVT = C * C / VEC;
    static constexpr int PK = (NVK + THREADS - 1) / THREADS;
    static constexpr int PV = (NVV + THREADS - 1) / THREADS;
    static constexpr int PT = (NVT + THREADS - 1) / THREADS;
    static constexpr int BYTES =
        (3 * C * LDK + DVT * LDK + C * LDV + 2 * DVT * LDC + 2 * C * LDC + C * LDV) *
            (int)sizeof(E) +
        3 * C * (int)sizeof(float);
};

template <typename E, int DK, int DVT, int C>
__global__ __launch_bounds__(512) void state_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const void* __restrict__ a, bool gate_bf16, const E* __restrict__ w,
    const E* __restrict__ Tm, const float* S0, E* __restrict__ o, float* S_T, int T, int DV,
    int NC) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int LDK = G::LDK, LDC = G::LDC, LDV = G::LDV, VEC = G::VEC;
    constexpr int BT = G::BT, BV = G::BV, BI = G::BI, BVA = G::BVA;
    constexpr int NTB = G::NTB, NVB = G::NVB, NT = G::NT;
    __shared__ __align__(16) E sK[C * LDK];
    __shared__ __align__(16) E sW[C * LDK];
    __shared__ __align__(16) E sQ[C * LDK];
    __shared__ __align__(16) E sS[DVT * LDK];  // state tile S[j][i] as an operand
    __shared__ __align__(16) E sR[C * LDV];    // R [t][j]
    __shared__ __align__(16) E sU[DVT * LDC];  // U^T [j][t]
    __shared__ __align__(16) E sUs[DVT * LDC]; // U^T scaled by gamma_C / gamma_t
    __shared__ __align__(16) E sT[C * LDC];    // (I + A)^{-1}  [t][s]
    __shared__ __align__(16) E sM[C * LDC];    // tril(Q W^T) * Gamma  [t][s]
    __shared__ __align__(16) E sV[C * LDV];
    __shared__ __align__(16) float sg[C];      // g_t (base 2)
    __shared__ __align__(16) float sgam[C];    // gamma_t = 2^g_t
    __shared__ __align__(16) float sdel[C];    // gamma_C / gamma_t

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t bh = blockIdx.y;
    const int j0 = blockIdx.x * DVT;

    // ---- registers holding the next chunk while the current one is computed
    uint4 pk[G::PK], pw[G::PK], pq[G::PK], pv[G::PV], pt[G::PT];
    float pa = 1.f;
    auto prefetch = [&](int c) {
        // rows past the end of the sequence load the last valid row and are
        // then zeroed, so that every load is unconditional
        const int t0 = c * C, n = min(C, T - t0);
        const size_t row0 = bh * T + t0;
#pragma unroll
        for (int x = 0; x < G::PK; ++x) {
            const int e = tid + G::THREADS * x;
            if (e < G::NVK) {
                const int t = e / (DK / VEC), c0 = (e % (DK / VEC)) * VEC;
                const size_t off = (row0 + min(t, n - 1)) * DK + c0;
                pk[x] = *reinterpret_cast<const uint4*>(k + off);
                pq[x] = *reinterpret_cast<const uint4*>(q + off);
                pw[x] = *reinterpret_cast<const uint4*>(w + off);
                if (t >= n) pk[x] = pq[x] = pw[x] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int x = 0; x < G::PV; ++x) {
            const int e = tid + G::THREADS * x;
            if (e < G::NVV) {
                const int t = e / (DVT / VEC), c0 = (e % (DVT / VEC)) * VEC;
                pv[x] = *reinterpret_cast<const uint4*>(v + (row0 + min(t, n - 1)) * DV + j0 + c0);
                if (t >= n) pv[x] = make_uint4(0, 0, 0, 0);
            }
        }
        const E* Tc = Tm + (bh * NC + c) * (size_t)(C * C);
#pragma unroll
        for (int x = 0; x < G::PT; ++x) {
            const int e = tid + G::THREADS * x;
            if (e < G::NVT) pt[x] = *reinterpret_cast<const uint4*>(Tc + e * VEC);
        }
        if (wave == 0) {
            pa = load_gate(a, row0 + min(lane, n - 1), gate_bf16);
            if (lane >= n) pa = 1.f;
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int x = 0; x < G::PK; ++x) {
            const int e = tid + G::THREADS * x;
            if (e < G::NVK) {
                const int t = e / (DK / VEC), c0 = (e % (DK / VEC)) * VEC;
                *reinterpret_cast<uint4*>(sK + t * LDK + c0) = pk[x];
                *reinterpret_cast<uint4*>(sQ + t * LDK + c0) = pq[x];
                *reinterpret_cast<uint4*>(sW + t * LDK + c0) = pw[x];
            }
        }
#pragma unroll
        for (int x = 0; x < G::PV; ++x) {
            const int e = tid + G::THREADS * x;
            if (e < G::NVV) {
                const int t = e / (DVT / VEC), c0 = (e % (DVT / VEC)) * VEC;
                *reinterpret_cast<uint4*>(sV + t * LDV + c0) = pv[x];
            }
        }
#pragma unroll
        for (int x = 0; x < G::PT; ++x) {
            const int e = tid + G::THREADS * x;
            if (e < G::NVT) {
                const int t = e / (C / VEC), c0 = (e % (C / VEC)) * VEC;
                *reinterpret_cast<uint4*>(sT + t * LDC + c0) = pt[x];
            }
        }
        if (wave == 0) {
            const float g = wave_incl_sum(lane < C ? log2_hw(pa) : 0.f);
            const float glast = lane_value(g, C - 1);
            if (lane < C) {
                sg[lane] = g;
                sgam[lane] = exp2_hw(g);
                sdel[lane] = exp2_hw(glast - g);
            }
        }
    };

    // ---- state: S^T blocks (BI x BV tiles), element e <-> i = 16 ti + 4 (lane/16) + e,
    //      j = 16 tj + lane % 16
    floatx4 accS[G::SPW][BI][BV];
#pragma unroll
    for (int x = 0; x < G::SPW; ++x) {
        const int job = wave + G::NW * x;
        const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bv = 0; bv < BV; ++bv) {
                accS[x][bi][bv] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (job < G::NSJ && S0) {
                    const int i = 16 * (ib + bi) + 4 * (lane >> 4);
                    const int j = 16 * (jb + bv) + (lane & 15);
                    const float4 s4 =
                        *reinterpret_cast<const float4*>(S0 + (bh * DV + j0 + j) * DK + i);
                    accS[x][bi][bv] = floatx4{s4.x, s4.y, s4.z, s4.w};
                }
            }
    }
    auto write_state = [&]() {
#pragma unroll
        for (int x = 0; x < G::SPW; ++x) {
            const int job = wave + G::NW * x;
            if (job < G::NSJ) {
                const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bv = 0; bv < BV; ++bv) {
                        const int i = 16 * (ib + bi) + 4 * (lane >> 4);
                        const int j = 16 * (jb + bv) + (lane & 15);
                        const floatx4 sv = accS[x][bi][bv];
                        store4<E>(sS + j * LDK + i, sv[0], sv[1], sv[2], sv[3]);
                    }
            }
        }
    };

    if (NC > 0) {
        prefetch(0);
        stage();
    }
    write_state();
    sync_lds();

    for (int c = 0; c < NC; ++c) {
        const int t0 = c * C, n = min(C, T - t0);
        const size_t row0 = bh * T + t0;
        if (c + 1 < NC) prefetch(c + 1);

        // ---------------- phase A: X^T = S K^T -> R ;  Y = S Q^T
        // block (jb: BVA j-tiles, tb: one t-tile); C-layout element e <->
        // j = 16 (jb + bv) + 4 (lane/16) + e, t = 16 tb + lane % 16
        floatx4 accY[G::APW][BVA][1];
#pragma unroll
        for (int x = 0; x < G::APW; ++x) {
            const int job = wave + G::NW * x;
            const int jb = (job / NT) * BVA, tb = job % NT;
            floatx4 xt[BVA][1];
#pragma unroll
            for (int bv = 0; bv < BVA; ++bv) {
                xt[bv][0] = floatx4{0.f, 0.f, 0.f, 0.f};
                accY[x][bv][0] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
            if (job < G::NAJ) {
                using M = Mma<E>;
                for (int kk = 0; kk < DK; kk += M::KS) {
                    typename M::frag_t fs[BVA];
#pragma unroll
                    for (int bv = 0; bv < BVA; ++bv)
                        fs[bv] = M::frag(sS, LDK, 16 * (jb + bv), kk, lane);
                    const auto fk = M::frag(sK, LDK, 16 * tb, kk, lane);
                    const auto fq = M::frag(sQ, LDK, 16 * tb, kk, lane);
#pragma unroll
                    for (int bv = 0; bv < BVA; ++bv) {
                        xt[bv][0] = M::mma(fs[bv], fk, xt[bv][0]);
                        accY[x][bv][0] = M::mma(fs[bv], fq, accY[x][bv][0]);
                    }
                }
                const int t = 16 * tb + (lane & 15);
                const float gt = sgam[t];
#pragma unroll
                for (int bv = 0; bv < BVA; ++bv) {
                    const int j = 16 * (jb + bv) + 4 * (lane >> 4);
                    float vv[4];
                    load4<E>(sV + t * LDV + j, vv);
                    const floatx4 xv = xt[bv][0];
                    store4<E>(sR + t * LDV + j, vv[0] - gt * xv[0], vv[1] - gt * xv[1],
                              vv[2] - gt * xv[2], vv[3] - gt * xv[3]);
                    accY[x][bv][0] = accY[x][bv][0] * gt;
                }
            }
        }
        sync_lds();

        // ---------------- phase B
        if (wave < 4) {
            // U = T R (T lower triangular: contract only up to the block's last row)
#pragma unroll
            for (int x = 0; x < G::UPW; ++x) {
                const int job = wave + 4 * x;
                if (job < G::NUJ) {
                    const int tb = (job / NVB) * BT, jb = (job % NVB) * BV;
                    floatx4 u[BT][BV];
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt)
#pragma unroll
                        for (int bv = 0; bv < BV; ++bv) u[bt][bv] = floatx4{0.f, 0.f, 0.f, 0.f};
                    mma_block<E, BT, BV, false, true>(u, sT, LDC, 16 * tb, sR, LDV, 16 * jb, 0,
                                                      16 * (tb + BT), lane);
#pragma unroll
                    for (int bt = 0; bt < BT; ++bt) {
                        const int t = 16 * (tb + bt) + 4 * (lane >> 4);
                        const float4 d4 = *reinterpret_cast<const float4*>(sdel + t);
#pragma unroll
                        for (int bv = 0; bv < BV; ++bv) {
                            const int j = 16 * (jb + bv) + (lane & 15);
                            const floatx4 uv = u[bt][bv];
                            store4<E>(sU + j * LDC + t, uv[0], uv[1], uv[2], uv[3]);
                            store4<E>(sUs + j * LDC + t, d4.x * uv[0], d4.y * uv[1],
                                      d4.z * uv[2], d4.w * uv[3]);
                        }
                    }
                }
            }
        } else {
            // M^T = W Q^T on the lower block triangle, stored as M[t][s]
#pragma unroll
            for (int x = 0; x < G::MPW; ++x) {
                const int job = (wave - 4) + 4 * x;
                if (job < G::NMJ) {
                    int tbb = 0, sbb = job;
                    while (sbb > tbb) {
                        sbb -= tbb + 1;
                        ++tbb;
                    }
                    floatx4 m[BT][BT];
#pragma unroll
                    for (int i = 0; i < BT; ++i)
#pragma unroll
                        for (int j = 0; j < BT; ++j) m[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
                    mma_block<E, BT, BT>(m, sW, LDK, 16 * sbb * BT, sQ, LDK, 16 * tbb * BT, 0,
                                         DK, lane);
#pragma unroll
                    for (int bs = 0; bs < BT; ++bs)
#pragma unroll
                        for (int bt = 0; bt < BT; ++bt) {
                            const int s0 = 16 * (sbb * BT + bs) + 4 * (lane >> 4);
                            const int t = 16 * (tbb * BT + bt) + (lane & 15);
                            const float gt = sg[t];
                            const float4 gs = *reinterpret_cast<const float4*>(sg + s0);
                            const floatx4 mv = m[bs][bt];
                            store4<E>(sM + t * LDC + s0,
                                      (s0 + 0 <= t) ? exp2_hw(gt - gs.x) * mv[0] : 0.f,
                                      (s0 + 1 <= t) ? exp2_hw(gt - gs.y) * mv[1] : 0.f,
                                      (s0 + 2 <= t) ? exp2_hw(gt - gs.z) * mv[2] : 0.f,
                                      (s0 + 3 <= t) ? exp2_hw(gt - gs.w) * mv[3] : 0.f);
                        }
                }
            }
        }
        sync_lds();

        // ---------------- phase C: O^T += U^T M^T ;  state update
#pragma unroll
        for (int x = 0; x < G::APW; ++x) {
            const int job = wave + G::NW * x;
            if (job < G::NAJ) {
                const int jb = (job / NT) * BVA, tb = job % NT;
                mma_block<E, BVA, 1>(accY[x], sU, LDC, 16 * jb, sM, LDC, 16 * tb, 0,
                                     16 * (tb + 1), lane);
                const int t = 16 * tb + (lane & 15);
                if (t < n) {
#pragma unroll
                    for (int bv = 0; bv < BVA; ++bv) {
                        const int j = 16 * (jb + bv) + 4 * (lane >> 4);
                        const floatx4 ov = accY[x][bv][0];
                        store4<E>(o + (row0 + t) * DV + j0 + j, ov[0], ov[1], ov[2], ov[3]);
                    }
                }
            }
        }
        const float gC = sgam[C - 1];
#pragma unroll
        for (int x = 0; x < G::SPW; ++x) {
            const int job = wave + G::NW * x;
            if (job < G::NSJ) {
                const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bv = 0; bv < BV; ++bv) accS[x][bi][bv] = accS[x][bi][bv] * gC;
                // W^T fragments straight from the token-major W
                mma_block<E, BI, BV, true>(accS[x], sW, LDK, 16 * ib, sUs, LDC, 16 * jb, 0, C,
                                           lane);
            }
        }
        sync_lds();

        // ---------------- phase D
        if (c + 1 < NC) stage();
        write_state();
        sync_lds();
    }
    if (S_T) {
#pragma unroll
        for (int x = 0; x < G::SPW; ++x) {
            const int job = wave + G::NW * x;
            if (job < G::NSJ) {
                const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bv = 0; bv < BV; ++bv) {
                        const int i = 16 * (ib + bi) + 4 * (lane >> 4);
                        const int j = 16 * (jb + bv) + (lane & 15);
                        const floatx4 sv = accS[x][bi][bv];
                        *reinterpret_cast<float4*>(S_T + (bh * DV + j0 + j) * DK + i) =
                            make_float4(sv[0], sv[1], sv[2], sv[3]);
                    }
            }
        }
    }
}

// ---------------------------------------------------------------- dispatch
template <typename E, int DK, int DVT, int C>
constexpr bool state_fits() {
    return StateCfg<E, DK, DVT, C>::BYTES <= kLdsLimit;
}

// widest d_v tile (64 or 32, at most d_v) whose LDS footprint fits; 0 if none
template <typename E, int DK, int C>
int pick_dvt(int dv) {
    if (dv >= 64 && state_fits<E, DK, 64, C>()) return 64;
    if (state_fits<E, DK, 32, C>()) return 32;
    return 0;
}

template <typename E>
int dv_tile_e(int dk, int dv, int C) {
#define KDN_PICK(DK_, C_) \
    if (dk == DK_ && C == C_) return pick_dvt<E, DK_, C_>(dv);
#define KDN_PICK_C(DK_) KDN_PICK(DK_, 16) KDN_PICK(DK_, 32) KDN_PICK(DK_, 64)
    KDN_PICK_C(32) KDN_PICK_C(64) KDN_PICK_C(128)
#undef KDN_PICK_C
#undef KDN_PICK
    return 0;
}

int dv_tile(const Shape& s) {
    return s.qkv_bf16 ? dv_tile_e<bf16_t>(s.dk, s.dv, s.chunk)
                      : dv_tile_e<float>(s.dk, s.dv, s.chunk);
}

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
    if constexpr (state_fits<E, DK, DVT, C>()) {
        hipLaunchKernelGGL((state_kernel<E, DK, DVT, C>), dim3(s.dv / DVT, s.BH),
                           dim3(StateCfg<E, DK, DVT, C>::THREADS), 0, st,
                           static_cast<const E*>(q), static_cast<const E*>(k),
                           static_cast<const E*>(v), a, s.gate_bf16, static_cast<const E*>(w),
                           static_cast<const E*>(Tm), S0, static_cast<E*>(o), S_T, s.T, s.dv,
                           s.nc);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
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
    const int dvt = dv_tile(s);
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
    return dv_tile(s) > 0;
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
