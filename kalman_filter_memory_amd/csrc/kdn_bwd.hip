// kdn_bwd.hip -- backward pass of the chunkwise KDN layer.
//
// Gradients of L = <dO, o> + <dS_T, S_T> + <dlambda_T, lambda_T> with respect
// to q, k, v, a, nu, r, lambda0 and S0: what training the layer needs ("Kalman
// Delta Networks", English abstract: the variants are pretrained inside
// language models).  Reverse-mode differentiation of the chunkwise forward of
// kdn_chunk.hip (ai-feeds.com summary, section 方法 step 3), in its notation:
// within a chunk with start state S, gamma_t = 2^(g_t), Gamma_ts = 2^(g_t - g_s),
// D_s = gamma_C / gamma_s,
//   A = strict_tril(K W^T * Gamma), T = (I + A)^{-1}, R = V - diag(gamma) K S^T,
//   U = T R, M = tril(Q W^T * Gamma), O = diag(gamma) Q S^T + M U,
//   S' = gamma_C S + U^T diag(D) W.
// With dS' the adjoint of the chunk-end state:
//   dU = diag(D) W dS'^T + M^T dO,      dR = T^T dU   (= dV)
//   dS = gamma_C dS' + dO^T diag(gamma) Q - dR^T diag(gamma) K
//   dM = tril(dO U^T),                   dA = -strict_tril(dR U^T)
//   dQ = diag(gamma) dO S + (dM * Gamma) W
//   dK = -diag(gamma) dR S + (dA * Gamma) W          (+ the gain's part)
//   dW = diag(D) U dS' + (dM * Gamma)^T Q + (dA * Gamma)^T K
// The decay enters through gamma, Gamma and D; its derivative is collected per
// token with respect to g_t (ln 2 cancels against the base-2 logarithm of a)
// and summed over the later tokens of the chunk to give d(ln a_t).
// The gain and the precision recursion ("Kalman Delta Networks", English
// abstract: Diagonal KDN, a Moebius-map uncertainty recurrence) are
// differentiated in variance form, per key dimension i (the isotropic
// variant's single chain is described at bgain_iso_kernel):
//   P^- = a^2 P + nu,  P = P^- / (1 + b P^-),  b = k_i^2 / r,
//   w_i = P^-_i k_i / D,  D = r + sum_j k_j^2 P^-_j.
// With G the adjoint of P after a token and s = sum_i dW_i w_i:
//   H  = (k_i / D)(dW_i - k_i s) + G (P / P^-)^2      (adjoint of P^-)
//   dk_i += (P^-_i / D)(dW_i - 2 k_i s) - G P^2 2 k_i / r
//   dnu += H,  da += 2 a P_prev H,  dr += -s / D + G P^2 b / r,  G <- a^2 H.
// G's recursion is affine, so it runs chunk-parallel: each chunk's map
// G_in = alpha G_out + beta, a carry over the chunks, then the outputs.
//
// Kernels, after a forward recompute that also keeps the state at every chunk
// start and 1/D of every token:
//   bstate_kernel  one workgroup per (head, d_v tile), chunks in reverse: dU,
//                  dR, the state adjoint (kept at every chunk end), dS0
//   bgrad_kernel   one workgroup per chunk, all chunks in parallel, over d_v
//                  slices: dQ, the memory part of dK, dW, s and d(ln a)
//   bgain_kernel   one workgroup per chunk: the precision recursion walked
//                  forward, then backward (alpha, beta; or, given G_out, the
//                  outputs); bgain_carry between the two
// All products on MFMA with fp32 accumulation; operands in the input dtype.
#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_tiles.h"

namespace kdn {
namespace {

constexpr int kLdsCap = 160 * 1024;
constexpr int kBThreads = 512;

// lower-triangular tile pair (tt >= ss) of triangle index j (row by row)
__device__ __forceinline__ void tri_pair(int j, int& tt, int& ss) {
    tt = 0;
    while ((tt + 1) * (tt + 2) / 2 <= j) ++tt;
    ss = j - tt * (tt + 1) / 2;
}

// ROWS x COLS of E from global rows of stride gld into LDS rows of stride sld
// with 16-byte vectors, in two steps through registers: the loads (rows >= n
// repeat row n - 1) issued ahead of the work they overlap, the stores (rows
// >= n zero) when the LDS buffer is free again.
template <typename E, int ROWS, int COLS> struct RegTile {
    static constexpr int V = Vec16<E>::N, VPR = COLS / V, NV = ROWS * VPR;
    static constexpr int IT = (NV + kBThreads - 1) / kBThreads;
};
template <typename E, int ROWS, int COLS> using TileRegs = u32x4[RegTile<E, ROWS, COLS>::IT];
template <typename E, int ROWS, int COLS>
__device__ __forceinline__ void tile_load(TileRegs<E, ROWS, COLS>& r, const E* src,
                                          size_t gld, int n, int tid) {
    using TT = RegTile<E, ROWS, COLS>;
#pragma unroll
    for (int x = 0; x < TT::IT; ++x) {
        const int e = tid + kBThreads * x;
        if (TT::NV % kBThreads == 0 || e < TT::NV) {
            const int t = e / TT::VPR, c0 = (e % TT::VPR) * TT::V;
            r[x] = *reinterpret_cast<const u32x4*>(src + min(t, n - 1) * gld + c0);
        }
    }
}
template <typename E, int ROWS, int COLS>
__device__ __forceinline__ void tile_store(E* dst, int sld, const TileRegs<E, ROWS, COLS>& r,
                                           int n, int tid) {
    using TT = RegTile<E, ROWS, COLS>;
#pragma unroll
    for (int x = 0; x < TT::IT; ++x) {
        const int e = tid + kBThreads * x;
        if (TT::NV % kBThreads == 0 || e < TT::NV) {
            const int t = e / TT::VPR, c0 = (e % TT::VPR) * TT::V;
            const u32x4 z = {0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(dst + t * sld + c0) = t < n ? r[x] : z;
        }
    }
}
template <int ROWS, int COLS> struct RegFTile {
    static constexpr int VPR = COLS / 4, NV = ROWS * VPR;
    static constexpr int IT = (NV + kBThreads - 1) / kBThreads;
};
template <int ROWS, int COLS> using FTileRegs = float4[RegFTile<ROWS, COLS>::IT];
template <int ROWS, int COLS>
__device__ __forceinline__ void ftile_load(FTileRegs<ROWS, COLS>& r, const float* src,
                                           size_t gld, int n, int tid) {
    using TT = RegFTile<ROWS, COLS>;
#pragma unroll
    for (int x = 0; x < TT::IT; ++x) {
        const int e = tid + kBThreads * x;
        if (TT::NV % kBThreads == 0 || e < TT::NV) {
            const int t = e / TT::VPR, c0 = (e % TT::VPR) * 4;
            r[x] = *reinterpret_cast<const float4*>(src + min(t, n - 1) * gld + c0);
        }
    }
}
template <typename E, int ROWS, int COLS>
__device__ __forceinline__ void ftile_store(E* dst, int sld, const FTileRegs<ROWS, COLS>& r,
                                            int n, int tid) {
    using TT = RegFTile<ROWS, COLS>;
#pragma unroll
    for (int x = 0; x < TT::IT; ++x) {
        const int e = tid + kBThreads * x;
        if (TT::NV % kBThreads == 0 || e < TT::NV) {
            const int t = e / TT::VPR, c0 = (e % TT::VPR) * 4;
            const float4 v = t < n ? r[x] : make_float4(0.f, 0.f, 0.f, 0.f);
            store4<E>(dst + t * sld + c0, v.x, v.y, v.z, v.w);
        }
    }
}

// dot product of two 16-byte vectors of E
template <typename E> __device__ __forceinline__ float dot16(u32x4 x, u32x4 y);
template <> __device__ __forceinline__ float dot16<float>(u32x4 x, u32x4 y) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fmaf(__uint_as_float(x[j]), __uint_as_float(y[j]), s);
    return s;
}
template <> __device__ __forceinline__ float dot16<bf16_t>(u32x4 x, u32x4 y) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s = fmaf(__uint_as_float(x[j] << 16), __uint_as_float(y[j] << 16), s);
        s = fmaf(__uint_as_float(x[j] & 0xFFFF0000u), __uint_as_float(y[j] & 0xFFFF0000u), s);
    }
    return s;
}

// sum over the 16 lanes of each 16-lane group (lanes sharing the rows of an
// MFMA result tile)
__device__ __forceinline__ float group16_sum(float x) {
    x += __shfl_xor(x, 1, kWave);
    x += __shfl_xor(x, 2, kWave);
    x += __shfl_xor(x, 4, kWave);
    x += __shfl_xor(x, 8, kWave);
    return x;
}

// The elements of a row-major LDS array X that lane l holds in a 16x16 MFMA
// result tile at (r0, c0): x[e] = X[r0 + 4 (l/16) + e][c0 + l % 16].  bfloat16:
// one transposing read (lane 4 j + p addresses row r0 + 4 (l/16) + j, columns
// c0 + 4 p .. + 3, and receives column c0 + l % 16 of the four rows).
template <typename E>
__device__ __forceinline__ void tile_col4(const E* X, int ld, int r0, int c0, int lane,
                                          float (&x)[4]);
template <>
__device__ __forceinline__ void tile_col4<bf16_t>(const bf16_t* X, int ld, int r0, int c0,
                                                  int lane, float (&x)[4]) {
    const short4x v =
        read_tr16(X + (r0 + 4 * (lane >> 4) + ((lane & 15) >> 2)) * ld + c0 + 4 * (lane & 3));
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = bf2f(static_cast<bf16_t>(v[e]));
}
template <>
__device__ __forceinline__ void tile_col4<float>(const float* X, int ld, int r0, int c0,
                                                 int lane, float (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = X[(r0 + 4 * (lane >> 4) + e) * ld + c0 + (lane & 15)];
}

// ======================================================= reverse state pass
template <typename E, int DK, int DVT, int C> struct BStateLds {
    using G = StateCfg<E, DK, DVT, C>;
    E K[C * G::LDK];
    E Q[C * G::LDK];
    E W[C * G::LDK];
    E dO[C * G::LDV];     // [t][j]; rows past the end are zero
    E Tt[C * G::LDC];     // T [t][s]
    E M[C * G::LDC];      // tril(Q W^T) * Gamma [t][s]
    E dUt[DVT * G::LDC];  // dU^T [j][s]
    E dOg[DVT * G::LDC];  // gamma_t dO[t][j] as [j][t]
    E dRg[DVT * G::LDC];  // -gamma_s dR[s][j] as [j][s]
    E S[DVT * G::LDK];    // the state adjoint as an operand [j][i]
    float g[C], gam[C], del[C];
};

template <typename E, int DK, int DVT, int C>
constexpr bool bstate_fits() {
    return sizeof(BStateLds<E, DK, DVT, C>) <= kLdsCap;
}

// One workgroup of 8 waves per (head, d_v tile), chunks from last to first.
// The state adjoint dS (S^T blocks, as the forward keeps S) lives in MFMA
// accumulators; per chunk:
//   1  dU = diag(D) W dS^T  (per wave: one s-tile x BVU j-tiles);  M tiles;
//      gamma-scaled transposed dO
//   2  dU += M^T dO, stored transposed
//   3  dR = T^T dU -> dv (fp32) and -gamma dR (transposed) for the update
//   4  dS <- gamma_C dS + Q^T (gamma dO) - K^T (gamma dR)
// The next chunk's operands are loaded into registers at the start of a chunk
// and staged at its end; the adjoint entering each chunk is stored (dSe).
template <typename E, int DK, int DVT, int C>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void bstate_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ dO,
    const float* __restrict__ gin, const E* __restrict__ w, const E* __restrict__ Tm,
    const float* __restrict__ dS_T, float* __restrict__ dv_out, E* __restrict__ dSe,
    float* __restrict__ dS0, int BH, int T, int DV, int NC) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int LDK = G::LDK, LDC = G::LDC, LDV = G::LDV, NT = G::NT, NV = G::NV;
    constexpr int BI = G::BI, BV = G::BV, NVB = G::NVB, VEC = G::VEC;
    constexpr int BVU = NV >= 2 ? 2 : 1, NUB = NV / BVU, NUJ = NT * NUB, UPW = (NUJ + 7) / 8;
    constexpr int NMT = NT * (NT + 1) / 2, MPW = (NMT + 7) / 8;
    __shared__ __align__(16) BStateLds<E, DK, DVT, C> L;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    // the d_v tiles of one head share an XCD (workgroups go to XCDs round-robin)
    const int ntile = DV / DVT, L_ = blockIdx.x, per = 8 * ntile;
    const int head = (L_ / per) * 8 + (L_ % 8);
    if (head >= BH) return;
    const size_t bh = head;
    const int j0 = ((L_ % per) / 8) * DVT;

    StateAcc<E, DK, DVT, C> acc;
#pragma unroll
    for (int x = 0; x < G::SPW; ++x) {
        const int job = wave + G::NW * x;
        const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bv = 0; bv < BV; ++bv) {
                acc[x][bi][bv] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (job < G::NSJ && dS_T) {
                    const int i = 16 * (ib + bi) + 4 * (lane >> 4);
                    const int j = 16 * (jb + bv) + (lane & 15);
                    const float4 s4 =
                        *reinterpret_cast<const float4*>(dS_T + (bh * DV + j0 + j) * DK + i);
                    acc[x][bi][bv] = floatx4{s4.x, s4.y, s4.z, s4.w};
                }
            }
    }

    u32x4 pk[G::PK], pq[G::PK], pw[G::PK], pv[G::PV], pt[G::PT];
    float pg = 0.f;
    // stage chunk cc from the registers; dO rows past the end are zeroed first
    auto stage = [&](int cc) {
        const int n = min(C, T - cc * C);
#pragma unroll
        for (int x = 0; x < G::PV; ++x) {
            const int e = tid + G::THREADS * x;
            if ((G::NVV % G::THREADS == 0 || e < G::NVV) && e / (DVT / VEC) >= n)
                pv[x] = u32x4{0u, 0u, 0u, 0u};
        }
        state_stage<E, DK, DVT, C, kStageAll>(L.K, L.Q, L.W, L.dO, L.Tt, L.g, L.gam, L.del, n,
                                              tid, lane, wave, pk, pq, pw, pv, pt, pg);
    };
    const Slab sl = slab_of<false>(bh, T, NC, Packed{});
    if (NC > 0) {
        state_prefetch<E, DK, DVT, C, kLoadAll>(q, k, dO, w, Tm, gin, sl, j0, DV, NC - 1, tid,
                                                lane, pk, pq, pw, pv, pt, pg);
        stage(NC - 1);
    }
    state_write<E, DK, DVT, C>(acc, L.S, wave, lane);
    sync_lds();

    for (int c = NC - 1; c >= 0; --c) {
        const int n = min(C, T - c * C);
        const size_t row0 = bh * T + (size_t)c * C;
        state_copy_out<E, DK, DVT, C>(L.S, dSe + ((bh * NC + c) * DV + j0) * DK, tid);
        if (c > 0)
            state_prefetch<E, DK, DVT, C, kLoadAll>(q, k, dO, w, Tm, gin, sl, j0, DV, c - 1, tid,
                                                    lane, pk, pq, pw, pv, pt, pg);
        // 1: dU = diag(D) W dS^T; M; gamma dO transposed
        floatx4 au[UPW][1][BVU];
#pragma unroll
        for (int x = 0; x < UPW; ++x) {
            const int job = wave + 8 * x;
#pragma unroll
            for (int bv = 0; bv < BVU; ++bv) au[x][0][bv] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (job < NUJ) {
                const int st = job / NUB, jb = (job % NUB) * BVU;
                mma_block<E, 1, BVU>(au[x], L.W, LDK, 16 * st, L.S, LDK, 16 * jb, 0, DK, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float d = L.del[16 * st + 4 * (lane >> 4) + e];
#pragma unroll
                    for (int bv = 0; bv < BVU; ++bv) au[x][0][bv][e] *= d;
                }
            }
        }
        // M tiles formed transposed (lane l: s = 16 ss + 4 (l/16) + e, t = 16 tt +
        // l % 16), so that each lane stores four consecutive s of a row t
#pragma unroll
        for (int x = 0; x < MPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NMT) {
                int tt, ss;
                tri_pair(job, tt, ss);
                const floatx4 m = mma_tile<E>(floatx4{0.f, 0.f, 0.f, 0.f}, L.W, LDK, 16 * ss, L.Q,
                                              LDK, 16 * tt, 0, DK, lane);
                const int t = 16 * tt + (lane & 15), s4 = 16 * ss + 4 * (lane >> 4);
                const float gt = L.g[t];
                float val[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    val[e] = s4 + e <= t ? m[e] * exp2_hw(gt - L.g[s4 + e]) : 0.f;
                store4<E>(L.M + t * LDC + s4, val[0], val[1], val[2], val[3]);
            }
        }
        // gamma_t dO[t][j] as [j][t]: per 16 x 16 tile, each lane reads four t of
        // a column j (one transposing read) and stores them as part of row j
#pragma unroll
        for (int x = 0; x < (NT * NV + 7) / 8; ++x) {
            const int job = wave + 8 * x;
            if (job < NT * NV) {
                const int tt = job / NV, jj = job % NV;
                float dv4[4];
                tile_col4<E>(L.dO, LDV, 16 * tt, 16 * jj, lane, dv4);
                const int t4 = 16 * tt + 4 * (lane >> 4);
                const float4 gm = *reinterpret_cast<const float4*>(L.gam + t4);
                store4<E>(L.dOg + (16 * jj + (lane & 15)) * LDC + t4, gm.x * dv4[0],
                          gm.y * dv4[1], gm.z * dv4[2], gm.w * dv4[3]);
            }
        }
        sync_lds();
        // 2: dU += M^T dO  (M[t][s] = 0 for t < s)
#pragma unroll
        for (int x = 0; x < UPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NUJ) {
                const int st = job / NUB, jb = (job % NUB) * BVU;
                mma_block<E, 1, BVU, true, true>(au[x], L.M, LDC, 16 * st, L.dO, LDV, 16 * jb,
                                                 16 * st, C, lane);
#pragma unroll
                for (int bv = 0; bv < BVU; ++bv) {
                    const int j = 16 * (jb + bv) + (lane & 15);
                    const floatx4 u = au[x][0][bv];
                    store4<E>(L.dUt + j * LDC + 16 * st + 4 * (lane >> 4), u[0], u[1], u[2], u[3]);
                }
            }
        }
        sync_lds();
        // 3: dR = T^T dU  (T[t][s] = 0 for t < s)
#pragma unroll
        for (int x = 0; x < UPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NUJ) {
                const int st = job / NUB, jb = (job % NUB) * BVU;
                floatx4 ar[1][BVU];
#pragma unroll
                for (int bv = 0; bv < BVU; ++bv) ar[0][bv] = floatx4{0.f, 0.f, 0.f, 0.f};
                mma_block<E, 1, BVU, true>(ar, L.Tt, LDC, 16 * st, L.dUt, LDC, 16 * jb, 16 * st,
                                           C, lane);
                const int s0 = 16 * st + 4 * (lane >> 4);
#pragma unroll
                for (int bv = 0; bv < BVU; ++bv) {
                    const int j = 16 * (jb + bv) + (lane & 15);
                    const floatx4 r4 = ar[0][bv];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (s0 + e < n) dv_out[(row0 + s0 + e) * DV + j0 + j] = r4[e];
                    store4<E>(L.dRg + j * LDC + s0, -L.gam[s0] * r4[0], -L.gam[s0 + 1] * r4[1],
                              -L.gam[s0 + 2] * r4[2], -L.gam[s0 + 3] * r4[3]);
                }
            }
        }
        sync_lds();
        // 4: dS <- gamma_C dS + Q^T (gamma dO) - K^T (gamma dR)
        const float gC = L.gam[C - 1];
#pragma unroll
        for (int x = 0; x < G::SPW; ++x) {
            const int job = wave + G::NW * x;
            if (job < G::NSJ) {
                const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
                for (int bi = 0; bi < BI; ++bi)
#pragma unroll
                    for (int bv = 0; bv < BV; ++bv) acc[x][bi][bv] = acc[x][bi][bv] * gC;
                mma_block<E, BI, BV, true>(acc[x], L.Q, LDK, 16 * ib, L.dOg, LDC, 16 * jb, 0, C,
                                           lane);
                mma_block<E, BI, BV, true>(acc[x], L.K, LDK, 16 * ib, L.dRg, LDC, 16 * jb, 0, C,
                                           lane);
            }
        }
        sync_lds();
        if (c > 0) stage(c - 1);
        state_write<E, DK, DVT, C>(acc, L.S, wave, lane);
        sync_lds();
    }
    if (dS0) {
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
                        const floatx4 sv = acc[x][bi][bv];
                        *reinterpret_cast<float4*>(dS0 + (bh * DV + j0 + j) * DK + i) =
                            make_float4(sv[0], sv[1], sv[2], sv[3]);
                    }
            }
        }
    }
}

// ===================================================== per-chunk gradients
template <typename E, int DK, int C, int JT> struct BGradLds {
    static constexpr int PAD = 32 / (int)sizeof(E);
    static constexpr int LDK = DK + PAD, LDC = C + PAD, LDJ = JT + PAD;
    E K[C * LDK];
    E Q[C * LDK];
    E W[C * LDK];
    E Tt[C * LDC];    // T; after the slices dM * Gamma  [t][s]
    E dAG[C * LDC];   // dA * Gamma [t][s]
    E Sj[JT * LDK];   // chunk-start state rows of the slice [j][i]
    E dSj[JT * LDK];  // chunk-end adjoint rows of the slice [j][i]
    E R[C * LDJ];     // V, then R = V - diag(gamma) K S^T  [t][j]
    E U[C * LDJ];     // [t][j]
    E dO[C * LDJ];    // [t][j]
    E dR[C * LDJ];    // [t][j]
    float g[C], gam[C], del[C];
    // per-wave partial sums, added in a fixed order at the end (no atomics:
    // the gradients are bitwise reproducible)
    float dlg[8][C], sdot[8][C], misc[8][2];
};

template <typename E, int DK, int C, int JT>
constexpr bool bgrad_fits() {
    return sizeof(BGradLds<E, DK, C, JT>) <= kLdsCap;
}

// One workgroup of 8 waves per chunk.  Over d_v slices of JT: R, U (recomputed
// from the chunk-start state), and the accumulation of dM, dA (lower-triangle
// tiles) and of gamma^-1 dQ1 = dO S, dR S and D^-1 dW1 = U dS' (per wave one
// t-tile x BKI i-tiles).  Then the decay derivative of every token, dM * Gamma
// and dA * Gamma, and the finished dQ, dK (memory part) and dW.
template <typename E, int DK, int C, int JT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void bgrad_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ dO, const float* __restrict__ dR, const E* __restrict__ w,
    const E* __restrict__ Tm, const float* __restrict__ gin, const E* __restrict__ Sc,
    const E* __restrict__ dSe, float* __restrict__ dq, float* __restrict__ dk,
    E* __restrict__ dW, float* __restrict__ sdot_out, float* __restrict__ dlna, int T, int DV,
    int NC) {
    using LL = BGradLds<E, DK, C, JT>;
    constexpr int LDK = LL::LDK, LDC = LL::LDC, LDJ = LL::LDJ;
    constexpr int NT = C / 16, NK = DK / 16, NJ = JT / 16;
    constexpr int BKI = NK >= 4 ? 4 : NK, NKB = NK / BKI, NQJ = NT * NKB, QPW = (NQJ + 7) / 8;
    constexpr int NMT = NT * (NT + 1) / 2, MPW = (NMT + 7) / 8;
    constexpr int BJX = NJ >= 2 ? 2 : 1, NXB = NJ / BJX, NXJ = NT * NXB, XPW = (NXJ + 7) / 8;
    __shared__ __align__(16) LL L;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int n = min(C, T - c * C);
    const size_t row0 = bh * T + (size_t)c * C;
    const size_t cidx = bh * NC + c;

    // every load of the chunk operands and of the first slice at once; the next
    // slice is loaded while the current one is worked on
    u32x4 rs[RegTile<E, JT, DK>::IT], rds[RegTile<E, JT, DK>::IT], rv[RegTile<E, C, JT>::IT],
        ro[RegTile<E, C, JT>::IT];
    float4 rr[RegFTile<C, JT>::IT];
    auto load_slice = [&](int j0) {
        tile_load<E, JT, DK>(rs, Sc + (cidx * DV + j0) * DK, DK, JT, tid);
        tile_load<E, JT, DK>(rds, dSe + (cidx * DV + j0) * DK, DK, JT, tid);
        tile_load<E, C, JT>(rv, v + row0 * DV + j0, DV, n, tid);
        tile_load<E, C, JT>(ro, dO + row0 * DV + j0, DV, n, tid);
        ftile_load<C, JT>(rr, dR + row0 * DV + j0, DV, n, tid);
    };
    float xc = 0.f;  // <dS', S> over the chunk state, from the staged registers
    auto store_slice = [&]() {
#pragma unroll
        for (int x = 0; x < RegTile<E, JT, DK>::IT; ++x) {
            const int e = tid + kBThreads * x;
            if (RegTile<E, JT, DK>::NV % kBThreads == 0 || e < RegTile<E, JT, DK>::NV)
                xc += dot16<E>(rs[x], rds[x]);
        }
        tile_store<E, JT, DK>(L.Sj, LDK, rs, JT, tid);
        tile_store<E, JT, DK>(L.dSj, LDK, rds, JT, tid);
        tile_store<E, C, JT>(L.R, LDJ, rv, n, tid);
        tile_store<E, C, JT>(L.dO, LDJ, ro, n, tid);
        ftile_store<E, C, JT>(L.dR, LDJ, rr, n, tid);
    };
    {
        u32x4 rk[RegTile<E, C, DK>::IT], rq[RegTile<E, C, DK>::IT], rw[RegTile<E, C, DK>::IT],
            rt[RegTile<E, C, C>::IT];
        tile_load<E, C, DK>(rk, k + row0 * DK, DK, n, tid);
        tile_load<E, C, DK>(rq, q + row0 * DK, DK, n, tid);
        tile_load<E, C, DK>(rw, w + row0 * DK, DK, n, tid);
        tile_load<E, C, C>(rt, Tm + cidx * C * C, C, C, tid);
        load_slice(0);
        tile_store<E, C, DK>(L.K, LDK, rk, n, tid);
        tile_store<E, C, DK>(L.Q, LDK, rq, n, tid);
        tile_store<E, C, DK>(L.W, LDK, rw, n, tid);
        tile_store<E, C, C>(L.Tt, LDC, rt, C, tid);
    }
    store_slice();
    if (tid < C) {
        const float gv = gin[cidx * C + tid], gC = gin[cidx * C + C - 1];
        L.g[tid] = gv;
        L.gam[tid] = exp2_hw(gv);
        L.del[tid] = exp2_hw(gC - gv);
#pragma unroll
        for (int w8 = 0; w8 < 8; ++w8) {
            L.dlg[w8][tid] = 0.f;
            L.sdot[w8][tid] = 0.f;
        }
        if (tid < 16) L.misc[tid >> 1][tid & 1] = 0.f;
    }

    floatx4 aq[QPW][1][BKI], ak[QPW][1][BKI], aw[QPW][1][BKI];
#pragma unroll
    for (int x = 0; x < QPW; ++x)
#pragma unroll
        for (int b = 0; b < BKI; ++b) {
            aq[x][0][b] = floatx4{0.f, 0.f, 0.f, 0.f};
            ak[x][0][b] = floatx4{0.f, 0.f, 0.f, 0.f};
            aw[x][0][b] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    floatx4 am[MPW], aa[MPW];
#pragma unroll
    for (int x = 0; x < MPW; ++x) {
        am[x] = floatx4{0.f, 0.f, 0.f, 0.f};
        aa[x] = floatx4{0.f, 0.f, 0.f, 0.f};
    }

    sync_lds();
    for (int j0 = 0; j0 < DV; j0 += JT) {
        const bool more = j0 + JT < DV;
        if (more) load_slice(j0 + JT);
        // R = V - diag(gamma) K S^T, in place
#pragma unroll
        for (int x = 0; x < XPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NXJ) {
                const int tt = job / NXB, jb = (job % NXB) * BJX;
                floatx4 ax[1][BJX];
#pragma unroll
                for (int b = 0; b < BJX; ++b) ax[0][b] = floatx4{0.f, 0.f, 0.f, 0.f};
                mma_block<E, 1, BJX>(ax, L.K, LDK, 16 * tt, L.Sj, LDK, 16 * jb, 0, DK, lane);
                // each lane rewrites only the elements of V it read itself
                const int t4 = 16 * tt + 4 * (lane >> 4);
                const float4 gm4 = *reinterpret_cast<const float4*>(L.gam + t4);
                const float gm[4] = {gm4.x, gm4.y, gm4.z, gm4.w};
#pragma unroll
                for (int b = 0; b < BJX; ++b) {
                    float vv[4];
                    tile_col4<E>(L.R, LDJ, 16 * tt, 16 * (jb + b), lane, vv);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        L.R[(t4 + e) * LDJ + 16 * (jb + b) + (lane & 15)] =
                            from_f<E>(vv[e] - gm[e] * ax[0][b][e]);
                }
            }
        }
        sync_lds();
        // U = T R  (T[t][s] = 0 for s > t)
#pragma unroll
        for (int x = 0; x < XPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NXJ) {
                const int tt = job / NXB, jb = (job % NXB) * BJX;
                // formed transposed, U^T = R^T T^T (lane l: j = 4 (l/16) + e, t = l % 16),
                // so that each lane stores four consecutive j of a row of U
                floatx4 au[BJX][1];
#pragma unroll
                for (int b = 0; b < BJX; ++b) au[b][0] = floatx4{0.f, 0.f, 0.f, 0.f};
                mma_block<E, BJX, 1, true, false>(au, L.R, LDJ, 16 * jb, L.Tt, LDC, 16 * tt, 0,
                                                  16 * (tt + 1), lane);
                const int t = 16 * tt + (lane & 15);
#pragma unroll
                for (int b = 0; b < BJX; ++b) {
                    const floatx4 uv = au[b][0];
                    store4<E>(L.U + t * LDJ + 16 * (jb + b) + 4 * (lane >> 4), uv[0], uv[1], uv[2],
                              uv[3]);
                }
            }
        }
        sync_lds();
        // dM^T += U dO^T, dA'^T += U dR^T (dA' negated later), transposed so that a
        // lane holds four consecutive s of one row t; dO S, dR S, U dS'
#pragma unroll
        for (int x = 0; x < MPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NMT) {
                int tt, ss;
                tri_pair(job, tt, ss);
                am[x] = mma_tile<E>(am[x], L.U, LDJ, 16 * ss, L.dO, LDJ, 16 * tt, 0, JT, lane);
                aa[x] = mma_tile<E>(aa[x], L.U, LDJ, 16 * ss, L.dR, LDJ, 16 * tt, 0, JT, lane);
            }
        }
#pragma unroll
        for (int x = 0; x < QPW; ++x) {
            const int job = wave + 8 * x;
            if (job < NQJ) {
                const int tt = job / NKB, ib = (job % NKB) * BKI;
                mma_block<E, 1, BKI, false, true>(aq[x], L.dO, LDJ, 16 * tt, L.Sj, LDK, 16 * ib,
                                                  0, JT, lane);
                mma_block<E, 1, BKI, false, true>(ak[x], L.dR, LDJ, 16 * tt, L.Sj, LDK, 16 * ib,
                                                  0, JT, lane);
                mma_block<E, 1, BKI, false, true>(aw[x], L.U, LDJ, 16 * tt, L.dSj, LDK, 16 * ib,
                                                  0, JT, lane);
            }
        }
        sync_lds();
        if (more) {
            store_slice();
            sync_lds();
        }
    }

    // xc: <dS', S> over the whole chunk state
    {
        float xs = wave_sum(xc);
        if (lane == 0) L.misc[wave][1] = xs;
    }
    // dQ1 = diag(gamma) dO S, dK1 = -diag(gamma) dR S, dW1 = diag(D) U dS';
    // decay derivative: + q_t.dQ1_t + k_t.dK1_t - w_t.dW1_t, and sum_s w_s.dW1_s
    // for the last token
#pragma unroll
    for (int x = 0; x < QPW; ++x) {
        const int job = wave + 8 * x;
        if (job < NQJ) {
            const int tt = job / NKB, ib = (job % NKB) * BKI;
            float wsum = 0.f;
            // q, k and w at the lane's elements of the tiles
            float qv[BKI][4], kv[BKI][4], wv[BKI][4];
#pragma unroll
            for (int b = 0; b < BKI; ++b) {
                tile_col4<E>(L.Q, LDK, 16 * tt, 16 * (ib + b), lane, qv[b]);
                tile_col4<E>(L.K, LDK, 16 * tt, 16 * (ib + b), lane, kv[b]);
                tile_col4<E>(L.W, LDK, 16 * tt, 16 * (ib + b), lane, wv[b]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tt + 4 * (lane >> 4) + e;
                const float gt = L.gam[t], dt = L.del[t];
                float row = 0.f, roww = 0.f;
#pragma unroll
                for (int b = 0; b < BKI; ++b) {
                    aq[x][0][b][e] *= gt;
                    ak[x][0][b][e] *= -gt;
                    aw[x][0][b][e] *= dt;
                    row += qv[b][e] * aq[x][0][b][e] + kv[b][e] * ak[x][0][b][e];
                    roww += wv[b][e] * aw[x][0][b][e];
                }
                row = group16_sum(row - roww);
                roww = group16_sum(roww);
                if ((lane & 15) == 0) L.dlg[wave][t] += row;
                wsum += roww;
            }
            wsum += __shfl_xor(wsum, 16, kWave);
            wsum += __shfl_xor(wsum, 32, kWave);
            if (lane == 0) L.misc[wave][0] += wsum;
        }
    }
    // M and A tiles, transposed like dM and dA (lane l: s = 16 ss + 4 (l/16) + e,
    // t = 16 tt + l % 16); dM * Gamma and dA * Gamma stored as rows t, four
    // consecutive s per lane; decay derivative: for each pair (t, s) of M (and
    // A), z = dM_ts M_ts adds to token t and subtracts from s
#pragma unroll
    for (int x = 0; x < MPW; ++x) {
        const int job = wave + 8 * x;
        if (job < NMT) {
            int tt, ss;
            tri_pair(job, tt, ss);
            const floatx4 mq = mma_tile<E>(floatx4{0.f, 0.f, 0.f, 0.f}, L.W, LDK, 16 * ss, L.Q,
                                           LDK, 16 * tt, 0, DK, lane);
            const floatx4 mk = mma_tile<E>(floatx4{0.f, 0.f, 0.f, 0.f}, L.W, LDK, 16 * ss, L.K,
                                           LDK, 16 * tt, 0, DK, lane);
            const int t = 16 * tt + (lane & 15), s4 = 16 * ss + 4 * (lane >> 4);
            const float gt = L.g[t];
            float row = 0.f, colz[4], vm[4], va[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = s4 + e;
                const float gm = s <= t ? exp2_hw(gt - L.g[s]) : 0.f;
                const float ga = s < t ? gm : 0.f;
                const float dm = am[x][e], dA = -aa[x][e];
                const float z = dm * mq[e] * gm + dA * mk[e] * ga;
                colz[e] = z;
                row += z;
                vm[e] = dm * gm;
                va[e] = dA * ga;
            }
            store4<E>(L.Tt + t * LDC + s4, vm[0], vm[1], vm[2], vm[3]);
            store4<E>(L.dAG + t * LDC + s4, va[0], va[1], va[2], va[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float zc = group16_sum(colz[e]);
                if ((lane & 15) == 0) L.dlg[wave][s4 + e] -= zc;
            }
            row += __shfl_xor(row, 16, kWave);
            row += __shfl_xor(row, 32, kWave);
            if (lane < 16) L.dlg[wave][t] += row;
        }
    }
    sync_lds();
    // dQ = dQ1 + (dM Gamma) W; dK = dK1 + (dA Gamma) W;
    // dW = dW1 + (dM Gamma)^T Q + (dA Gamma)^T K; s_t = dW_t . w_t
#pragma unroll
    for (int x = 0; x < QPW; ++x) {
        const int job = wave + 8 * x;
        if (job < NQJ) {
            const int tt = job / NKB, ib = (job % NKB) * BKI;
            mma_block<E, 1, BKI, false, true>(aq[x], L.Tt, LDC, 16 * tt, L.W, LDK, 16 * ib, 0,
                                              16 * (tt + 1), lane);
            mma_block<E, 1, BKI, false, true>(ak[x], L.dAG, LDC, 16 * tt, L.W, LDK, 16 * ib, 0,
                                              16 * (tt + 1), lane);
            mma_block<E, 1, BKI, true, true>(aw[x], L.Tt, LDC, 16 * tt, L.Q, LDK, 16 * ib,
                                             16 * tt, C, lane);
            mma_block<E, 1, BKI, true, true>(aw[x], L.dAG, LDC, 16 * tt, L.K, LDK, 16 * ib,
                                             16 * tt, C, lane);
            float wv[BKI][4];
#pragma unroll
            for (int b = 0; b < BKI; ++b)
                tile_col4<E>(L.W, LDK, 16 * tt, 16 * (ib + b), lane, wv[b]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tt + 4 * (lane >> 4) + e;
                float sd = 0.f;
#pragma unroll
                for (int b = 0; b < BKI; ++b) {
                    const int i = 16 * (ib + b) + (lane & 15);
                    // s_t from the unrounded dW (dW itself is stored in the input dtype)
                    const E dw = from_f<E>(aw[x][0][b][e]);
                    sd += aw[x][0][b][e] * wv[b][e];
                    if (t < n) {
                        const size_t o = (row0 + t) * DK + i;
                        dq[o] = aq[x][0][b][e];
                        dk[o] = ak[x][0][b][e];
                        dW[o] = dw;
                    }
                }
                sd = group16_sum(sd);
                if ((lane & 15) == 0) L.sdot[wave][t] += sd;
            }
        }
    }
    sync_lds();
    // d(ln a_t) = sum over the chunk's tokens u >= t of the derivative w.r.t. g_u;
    // the state carried to the next chunk adds gamma_C <dS', S> and
    // sum_s w_s.dW1_s to the last token
    if (wave == 0) {
        float x = 0.f, sd = 0.f, m0 = 0.f, m1 = 0.f;
        const int tl = min(lane, C - 1);
#pragma unroll
        for (int w8 = 0; w8 < 8; ++w8) {
            x += L.dlg[w8][tl];
            sd += L.sdot[w8][tl];
            m0 += L.misc[w8][0];
            m1 += L.misc[w8][1];
        }
        if (lane >= n) x = 0.f;
        if (lane == n - 1) x += m0 + L.gam[C - 1] * m1;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_down(x, off, kWave);
            if (lane + off < kWave) x += y;
        }
        if (lane < n) {
            dlna[row0 + lane] = x;
            sdot_out[row0 + lane] = sd;
        }
    }
}

// ============================================== gain and precision recursion
// One workgroup per chunk, lane i = key dimension.  The precision is walked
// forward from the chunk-boundary value (P^- kept in LDS), then backward:
//   APPLY = false: the chunk's affine map G_in = alpha G_out + beta (float2)
//   APPLY = true:  with G_out given, dk += the gain's part, and per token
//                  da = d(ln a)/a + sum_i 2 a P_prev H, dnu = sum_i H,
//                  dr = -s/D + sum_i G P^2 b / r.
template <typename E, typename G, int DK, int C, bool APPLY>
__global__ __launch_bounds__(DK < 64 ? 64 : DK) void bgain_kernel(
    const E* __restrict__ k, const G* __restrict__ a, const G* __restrict__ nu,
    const G* __restrict__ r, const float* __restrict__ lam_chunk, const float* __restrict__ dinv,
    const float* __restrict__ sdot, const E* __restrict__ dW, const float* __restrict__ dlna,
    const float* __restrict__ Gout, float2* __restrict__ ab, float* __restrict__ dk,
    float* __restrict__ da, float* __restrict__ dnu, float* __restrict__ dr, int T, int NC) {
    constexpr int NW = (DK < 64 ? 64 : DK) / 64;
    // per token and wave: sum_i H, sum_i 2 a P_prev H, sum_i G P^2 b/r (summed
    // over the waves in a fixed order at the end)
    __shared__ float red[NW][3][C];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int n = min(C, T - c * C);
    const size_t row0 = bh * T + (size_t)c * C;
    const int i = tid;
    const bool act = i < DK;
    const int ic = act ? i : 0;
    // token scalars in lane t (broadcast with readlane)
    const size_t tk = row0 + min(lane, n - 1);
    const float ta = to_f<G>(a[tk]), tnu = to_f<G>(nu[tk]), tr = to_f<G>(r[tk]);
    const float tir = 1.f / tr, tdi = dinv[tk], tsd = sdot[tk];
    const float tia = 1.f / ta;  // one division per token, not per (token, dimension)
    // forward: P^- of every token from the chunk-boundary precision
    float P = 1.f / lam_chunk[(bh * (NC + 1) + c) * DK + ic];
    float pms[C];  // P^- of every token (both walks fully unrolled: static indices)
#pragma unroll
    for (int g0 = 0; g0 < C; g0 += 16) {
        float kg[16];
#pragma unroll
        for (int h = 0; h < 16; ++h) kg[h] = to_f<E>(k[(row0 + min(g0 + h, n - 1)) * DK + ic]);
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            const int t = g0 + h;
            if (t < n) {
                const float at = lane_value(ta, t), nut = lane_value(tnu, t);
                const float irt = lane_value(tir, t);
                const float pm = fmaf(at * at, P, nut);
                pms[t] = pm;
                P = pm * rcp(fmaf(kg[h] * kg[h] * irt, pm, 1.f));
            }
        }
    }
    // backward over the tokens, 16 at a time (every load of a group issued at
    // its start; the gain's part of dk added to the memory part in registers)
    float al = 1.f, be = 0.f, Gv = 0.f;
    if constexpr (APPLY) Gv = act ? Gout[(bh * NC + c) * DK + i] : 0.f;
#pragma unroll
    for (int g0 = C - 16; g0 >= 0; g0 -= 16) {
        float kg[16], dwg[16], dkg[16], hv[16], ha[16], hr[16];
#pragma unroll
        for (int h = 0; h < 16; ++h) {
            const size_t o = (row0 + min(g0 + h, n - 1)) * DK + ic;
            kg[h] = to_f<E>(k[o]);
            dwg[h] = to_f<E>(dW[o]);
            if constexpr (APPLY) dkg[h] = dk[o];
        }
#pragma unroll
        for (int h = 15; h >= 0; --h) {
            const int t = g0 + h;
            hv[h] = 0.f;
            ha[h] = 0.f;
            hr[h] = 0.f;
            if (t < n) {
                const float at = lane_value(ta, t), nut = lane_value(tnu, t);
                const float irt = lane_value(tir, t), dit = lane_value(tdi, t);
                const float sdt = lane_value(tsd, t);
                const float kv = kg[h], pm = pms[t];
                const float b = kv * kv * irt;
                // P / P^- = 1 / (1 + b P^-): one reciprocal for both
                const float rat = rcp(fmaf(b, pm, 1.f)), c2 = rat * rat;
                const float Pt = pm * rat;
                const float gainP = kv * dit * (dwg[h] - kv * sdt);
                if constexpr (APPLY) {
                    const float H = fmaf(c2, Gv, gainP);
                    const float db = -Gv * Pt * Pt;
                    dkg[h] += pm * dit * (dwg[h] - 2.f * kv * sdt) + db * 2.f * kv * irt;
                    if (act) {
                        hv[h] = H;
                        ha[h] = 2.f * (pm - nut) * H * lane_value(tia, t);
                        hr[h] = -db * b * irt;
                    }
                    Gv = at * at * H;
                } else {
                    al = at * at * c2 * al;
                    be = at * at * fmaf(c2, be, gainP);
                }
            }
        }
        if constexpr (APPLY) {
            if (act) {
#pragma unroll
                for (int h = 0; h < 16; ++h)
                    if (g0 + h < n) dk[(row0 + g0 + h) * DK + i] = dkg[h];
            }
            // per-token sums over the key dimensions of these 16 tokens
            float sv = transpose_sum16(hv, lane), sa = transpose_sum16(ha, lane),
                  sr = transpose_sum16(hr, lane);
            sv += __shfl_xor(sv, 16, kWave);
            sv += __shfl_xor(sv, 32, kWave);
            sa += __shfl_xor(sa, 16, kWave);
            sa += __shfl_xor(sa, 32, kWave);
            sr += __shfl_xor(sr, 16, kWave);
            sr += __shfl_xor(sr, 32, kWave);
            if (lane < 16) {
                red[wave][0][g0 + lane] = sv;
                red[wave][1][g0 + lane] = sa;
                red[wave][2][g0 + lane] = sr;
            }
        }
    }
    if constexpr (!APPLY) {
        if (act) ab[(bh * NC + c) * DK + i] = make_float2(al, be);
    } else {
        __syncthreads();
        if (tid < n) {
            const size_t o = row0 + tid;
            float sv = 0.f, sa = 0.f, sr = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                sv += red[w][0][tid];
                sa += red[w][1][tid];
                sr += red[w][2][tid];
            }
            da[o] = dlna[o] / ta + sa;
            dnu[o] = sv;
            dr[o] = -tsd * tdi + sr;
        }
    }
}

// Isotropic variant: one precision per head, so the recursion is one scalar
// chain and every per-token quantity is a scalar; with kappa = |k|^2,
// b = kappa / (d_k r), D = P^- kappa + r, w = P^- k / D and s = dW . w:
//   H = s r / (P^- D) + G (P / P^-)^2,  dkappa = -P^- s / D - G P^2 / (d_k r),
//   dk += dW P^- / D + 2 dkappa k,  dr = -s / D + G P^2 b / r,
//   dnu = H,  da = d(ln a)/a + 2 a P_prev H,  G <- a^2 H.
// One workgroup of 4 waves per chunk: kappa by all threads, the chain on wave 0
// (lane t keeps token t), the dk update by all threads in 16-byte pieces.
template <typename E, typename G, int DK, int C, bool APPLY>
__global__ __launch_bounds__(256) void bgain_iso_kernel(
    const E* __restrict__ k, const G* __restrict__ a, const G* __restrict__ nu,
    const G* __restrict__ r, const float* __restrict__ lam_chunk, const float* __restrict__ sdot,
    const E* __restrict__ dW, const float* __restrict__ dlna, const float* __restrict__ Gout,
    float2* __restrict__ ab, float* __restrict__ dk, float* __restrict__ da,
    float* __restrict__ dnu, float* __restrict__ dr, int T, int NC) {
    __shared__ float skk[C], scA[C], scB[C];
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int c = blockIdx.x;
    const size_t bh = blockIdx.y;
    const int n = min(C, T - c * C);
    const size_t row0 = bh * T + (size_t)c * C;
    // kappa_t, four threads per token
    {
        constexpr int V = Vec16<E>::N, PER = DK / 4;
        const int t = tid >> 2, part = tid & 3;
        float acc = 0.f;
        if (t < C) {
            const E* row = k + (row0 + min(t, n - 1)) * DK + part * PER;
#pragma unroll
            for (int j = 0; j < PER; j += V) {
                const u32x4 x = *reinterpret_cast<const u32x4*>(row + j);
                acc += dot16<E>(x, x);
            }
        }
        acc += __shfl_xor(acc, 1, kWave);
        acc += __shfl_xor(acc, 2, kWave);
        if (t < C && part == 0) skk[t] = acc;
    }
    __syncthreads();
    if (wave == 0) {
        const size_t tk = row0 + min(lane, n - 1);
        const float ta = to_f<G>(a[tk]), tnu = to_f<G>(nu[tk]), tr = to_f<G>(r[tk]);
        const float tir = 1.f / tr, tsd = sdot[tk], tkk = skk[min(lane, C - 1)];
        const float tb = tkk * tir * (1.f / static_cast<float>(DK));
        // forward walk (the same on every lane); lane t keeps P^- of token t
        float P = 1.f / lam_chunk[bh * (NC + 1) + c], pml = 1.f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
            if (t < n) {
                const float at = lane_value(ta, t), pm = fmaf(at * at, P, lane_value(tnu, t));
                if (lane == t) pml = pm;
                P = pm * rcp(fmaf(lane_value(tb, t), pm, 1.f));
            }
        }
        const float iD = 1.f / fmaf(pml, tkk, tr);
        const float Pt = pml * rcp(fmaf(tb, pml, 1.f));
        const float rat = Pt * rcp(pml), c2 = rat * rat;
        const float gainP = tsd * tr * iD * rcp(pml);
        if constexpr (!APPLY) {
            float al = 1.f, be = 0.f;
#pragma unroll
            for (int t = C - 1; t >= 0; --t) {
                if (t < n) {
                    const float at = lane_value(ta, t), a2 = at * at;
                    al = a2 * lane_value(c2, t) * al;
                    be = a2 * fmaf(lane_value(c2, t), be, lane_value(gainP, t));
                }
            }
            if (lane == 0) ab[bh * NC + c] = make_float2(al, be);
        } else {
            float Gv = Gout[bh * NC + c], Gl = 0.f;
#pragma unroll
            for (int t = C - 1; t >= 0; --t) {
                if (t < n) {
                    if (lane == t) Gl = Gv;
                    const float at = lane_value(ta, t);
                    Gv = at * at * fmaf(lane_value(c2, t), Gv, lane_value(gainP, t));
                }
            }
            const float H = fmaf(c2, Gl, gainP), db = -Gl * Pt * Pt;
            const float dkap = -pml * tsd * iD + db * tir * (1.f / static_cast<float>(DK));
            if (lane < n) {
                da[tk] = dlna[tk] / ta + 2.f * (pml - tnu) * H / ta;
                dnu[tk] = H;
                dr[tk] = -tsd * iD - db * tb * tir;
                scA[lane] = pml * iD;
                scB[lane] = 2.f * dkap;
            }
        }
    }
    if constexpr (APPLY) {
        __syncthreads();
        // dk += dW P^- / D + 2 dkappa k, four components at a time
        for (int e = tid; e < n * (DK / 4); e += 256) {
            const int t = e / (DK / 4), i0 = (e % (DK / 4)) * 4;
            const size_t o = (row0 + t) * DK + i0;
            float kv[4], wv[4];
            load4<E>(k + o, kv);
            load4<E>(dW + o, wv);
            float4 d4 = *reinterpret_cast<const float4*>(dk + o);
            const float A = scA[t], B = scB[t];
            d4.x += fmaf(wv[0], A, B * kv[0]);
            d4.y += fmaf(wv[1], A, B * kv[1]);
            d4.z += fmaf(wv[2], A, B * kv[2]);
            d4.w += fmaf(wv[3], A, B * kv[3]);
            *reinterpret_cast<float4*>(dk + o) = d4;
        }
    }
}

// G_out of every chunk from the chunk maps, last chunk first; dlambda0 at the end
__global__ void bgain_carry_kernel(const float2* __restrict__ ab,
                                   const float* __restrict__ lam_chunk,
                                   const float* __restrict__ dlambda_T, float* __restrict__ Gout,
                                   float* __restrict__ dlambda0, int BH, int DK, int NC) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= BH * DK) return;
    const size_t bh = idx / DK;
    const int i = idx % DK;
    const float lT = lam_chunk[(bh * (NC + 1) + NC) * DK + i];
    float G = dlambda_T ? -dlambda_T[idx] * lT * lT : 0.f;
    // eight chunk maps loaded at a time, so the chain waits once per eight
    for (int c8 = NC - 1; c8 >= 0; c8 -= 8) {
        float2 m[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) m[u] = ab[(bh * NC + max(c8 - u, 0)) * DK + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (c8 - u >= 0) {
                Gout[(bh * NC + c8 - u) * DK + i] = G;
                G = fmaf(m[u].x, G, m[u].y);
            }
        }
    }
    if (dlambda0) {
        const float l0 = lam_chunk[bh * (NC + 1) * DK + i];
        // no tokens: lambda_T is lambda0 and its cotangent passes through as is
        dlambda0[idx] = NC == 0 ? (dlambda_T ? dlambda_T[idx] : 0.f) : -G / (l0 * l0);
    }
}

// ---------------------------------------------------------------- launchers
template <typename E, int DK, int DVT, int C>
hipError_t bstate_t(const Shape& s, const BwdArgs& b, hipStream_t st) {
    if constexpr (bstate_fits<E, DK, DVT, C>()) {
        const int groups = (s.BH + 7) / 8;
        launch_k((bstate_kernel<E, DK, DVT, C>), dim3(groups * 8 * (s.dv / DVT)), dim3(512), 0,
                 st, static_cast<const E*>(b.q), static_cast<const E*>(b.k),
                 static_cast<const E*>(b.dO), b.g, static_cast<const E*>(b.w),
                 static_cast<const E*>(b.Tm), b.dS_T, b.dv, static_cast<E*>(b.dSe), b.dS0, s.BH,
                 s.T, s.dv, s.nc);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <typename E, int DK, int C>
int bstate_tile(int dv) {
    if (dv >= 64 && bstate_fits<E, DK, 64, C>()) return 64;
    if (bstate_fits<E, DK, 32, C>()) return 32;
    return 0;
}

template <typename E, int DK, int C, int JT>
hipError_t bgrad_t(const Shape& s, const BwdArgs& b, hipStream_t st) {
    if constexpr (bgrad_fits<E, DK, C, JT>()) {
        launch_k((bgrad_kernel<E, DK, C, JT>), dim3(s.nc, s.BH), dim3(512), 0, st,
                 static_cast<const E*>(b.q), static_cast<const E*>(b.k),
                 static_cast<const E*>(b.v), static_cast<const E*>(b.dO), b.dv,
                 static_cast<const E*>(b.w), static_cast<const E*>(b.Tm), b.g,
                 static_cast<const E*>(b.Sc), static_cast<const E*>(b.dSe), b.dq, b.dk,
                 static_cast<E*>(b.dW), b.sdot, b.dlna, s.T, s.dv, s.nc);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <typename E, int DK, int C>
int bgrad_slice(int dv) {
    if (dv >= 64 && bgrad_fits<E, DK, C, 64>()) return 64;
    if (dv >= 32 && bgrad_fits<E, DK, C, 32>()) return 32;
    if (bgrad_fits<E, DK, C, 16>()) return 16;
    return 0;
}

template <typename E, typename G, int DK, int C>
hipError_t bgain_t(const Shape& s, const BwdArgs& b, hipStream_t st) {
    constexpr int NTH = DK < 64 ? 64 : DK;
    const dim3 grid(s.nc, s.BH);
    // a timing request covers the three launches: start at the first, stop at the last
    const LaunchTiming tm = launch_timing();
    launch_timing() = LaunchTiming{tm.start, nullptr};
    launch_k((bgain_kernel<E, G, DK, C, false>), grid, dim3(NTH), 0, st,
             static_cast<const E*>(b.k), static_cast<const G*>(b.a), static_cast<const G*>(b.nu),
             static_cast<const G*>(b.r), b.lam_chunk, b.dinv, b.sdot,
             static_cast<const E*>(b.dW), b.dlna, b.Gout,
             reinterpret_cast<float2*>(b.ab), b.dk, b.da, b.dnu, b.dr, s.T, s.nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = s.BH * s.dk;
    hipLaunchKernelGGL(bgain_carry_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                       reinterpret_cast<const float2*>(b.ab), b.lam_chunk, b.dlambda_T, b.Gout,
                       b.dlambda0, s.BH, s.dk, s.nc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_timing() = LaunchTiming{nullptr, tm.stop};
    launch_k((bgain_kernel<E, G, DK, C, true>), grid, dim3(NTH), 0, st,
             static_cast<const E*>(b.k), static_cast<const G*>(b.a), static_cast<const G*>(b.nu),
             static_cast<const G*>(b.r), b.lam_chunk, b.dinv, b.sdot,
             static_cast<const E*>(b.dW), b.dlna, b.Gout,
             reinterpret_cast<float2*>(b.ab), b.dk, b.da, b.dnu, b.dr, s.T, s.nc);
    return hipGetLastError();
}

template <typename E, typename G, int DK, int C>
hipError_t bgain_iso_t(const Shape& s, const BwdArgs& b, hipStream_t st) {
    const dim3 grid(s.nc, s.BH);
    const LaunchTiming tm = launch_timing();
    launch_timing() = LaunchTiming{tm.start, nullptr};
    launch_k((bgain_iso_kernel<E, G, DK, C, false>), grid, dim3(256), 0, st,
             static_cast<const E*>(b.k), static_cast<const G*>(b.a), static_cast<const G*>(b.nu),
             static_cast<const G*>(b.r), b.lam_chunk, b.sdot, static_cast<const E*>(b.dW),
             b.dlna, b.Gout, reinterpret_cast<float2*>(b.ab), b.dk, b.da, b.dnu, b.dr, s.T, s.nc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bgain_carry_kernel, dim3((s.BH + 255) / 256), dim3(256), 0, st,
                       reinterpret_cast<const float2*>(b.ab), b.lam_chunk, b.dlambda_T, b.Gout,
                       b.dlambda0, s.BH, 1, s.nc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch_timing() = LaunchTiming{nullptr, tm.stop};
    launch_k((bgain_iso_kernel<E, G, DK, C, true>), grid, dim3(256), 0, st,
             static_cast<const E*>(b.k), static_cast<const G*>(b.a), static_cast<const G*>(b.nu),
             static_cast<const G*>(b.r), b.lam_chunk, b.sdot, static_cast<const E*>(b.dW),
             b.dlna, b.Gout, reinterpret_cast<float2*>(b.ab), b.dk, b.da, b.dnu, b.dr, s.T, s.nc);
    return hipGetLastError();
}

template <typename E>
hipError_t bwd_state_e(const Shape& s, const BwdArgs& b, hipStream_t st) {
#define KDN_BS(DK_, DVT_, C_)                                                          \
    if (s.dk == DK_ && C_ == s.chunk && bstate_tile<E, DK_, C_>(s.dv) == DVT_ &&       \
        s.dv % DVT_ == 0)                                                              \
        return bstate_t<E, DK_, DVT_, C_>(s, b, st);
#define KDN_BS_C(DK_, DVT_) KDN_BS(DK_, DVT_, 16) KDN_BS(DK_, DVT_, 32) KDN_BS(DK_, DVT_, 64)
    KDN_BS_C(32, 32) KDN_BS_C(32, 64) KDN_BS_C(64, 32) KDN_BS_C(64, 64)
    KDN_BS_C(128, 32) KDN_BS_C(128, 64)
#undef KDN_BS_C
#undef KDN_BS
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t bwd_grad_e(const Shape& s, const BwdArgs& b, hipStream_t st) {
#define KDN_BG(DK_, C_, JT_)                                                           \
    if (s.dk == DK_ && C_ == s.chunk && bgrad_slice<E, DK_, C_>(s.dv) == JT_)          \
        return bgrad_t<E, DK_, C_, JT_>(s, b, st);
#define KDN_BG_C(DK_, C_) KDN_BG(DK_, C_, 16) KDN_BG(DK_, C_, 32) KDN_BG(DK_, C_, 64)
#define KDN_BG_K(DK_) KDN_BG_C(DK_, 16) KDN_BG_C(DK_, 32) KDN_BG_C(DK_, 64)
    KDN_BG_K(32) KDN_BG_K(64) KDN_BG_K(128)
#undef KDN_BG_K
#undef KDN_BG_C
#undef KDN_BG
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t bwd_gain_e(const Shape& s, const BwdArgs& b, hipStream_t st) {
#define KDN_BN(DK_, C_)                                                                \
    if (s.dk == DK_ && s.chunk == C_) {                                                \
        if (!s.diag)                                                                   \
            return s.gate_bf16 ? bgain_iso_t<E, bf16_t, DK_, C_>(s, b, st)             \
                               : bgain_iso_t<E, float, DK_, C_>(s, b, st);             \
        return s.gate_bf16 ? bgain_t<E, bf16_t, DK_, C_>(s, b, st)                     \
                           : bgain_t<E, float, DK_, C_>(s, b, st);                     \
    }
#define KDN_BN_C(DK_) KDN_BN(DK_, 16) KDN_BN(DK_, 32) KDN_BN(DK_, 64)
    KDN_BN_C(32) KDN_BN_C(64) KDN_BN_C(128)
#undef KDN_BN_C
#undef KDN_BN
    return hipErrorInvalidValue;
}

template <typename E>
bool bwd_supported_e(const Shape& s) {
    bool st = false, gr = false;
#define KDN_SUP(DK_, C_)                                                               \
    if (s.dk == DK_ && s.chunk == C_) {                                                \
        const int t = bstate_tile<E, DK_, C_>(s.dv);                                   \
        st = t > 0 && s.dv % t == 0;                                                   \
        gr = bgrad_slice<E, DK_, C_>(s.dv) > 0;                                        \
    }
#define KDN_SUP_C(DK_) KDN_SUP(DK_, 16) KDN_SUP(DK_, 32) KDN_SUP(DK_, 64)
    KDN_SUP_C(32) KDN_SUP_C(64) KDN_SUP_C(128)
#undef KDN_SUP_C
#undef KDN_SUP
    return st && gr;
}

}  // namespace

bool backward_supported(const Shape& s) {
    if (!chunk_supported(s)) return false;
    return s.qkv_bf16 ? bwd_supported_e<bf16_t>(s) : bwd_supported_e<float>(s);
}

hipError_t launch_bwd_state(const Shape& s, const BwdArgs& b, hipStream_t st) {
    if (s.BH == 0) return hipSuccess;
    return s.qkv_bf16 ? bwd_state_e<bf16_t>(s, b, st) : bwd_state_e<float>(s, b, st);
}

hipError_t launch_bwd_grad(const Shape& s, const BwdArgs& b, hipStream_t st) {
    if (s.BH == 0 || s.nc == 0) return hipSuccess;
    return s.qkv_bf16 ? bwd_grad_e<bf16_t>(s, b, st) : bwd_grad_e<float>(s, b, st);
}

hipError_t launch_bwd_gain(const Shape& s, const BwdArgs& b, hipStream_t st) {
    if (s.BH == 0) return hipSuccess;
    if (s.nc == 0) {
        // no tokens: dlambda0 = dlambda_T (the carry over zero chunks)
        const int nl = s.diag ? s.dk : 1, n = s.BH * nl;
        hipLaunchKernelGGL(bgain_carry_kernel, dim3((n + 255) / 256), dim3(256), 0, st,
                           reinterpret_cast<const float2*>(b.ab), b.lam_chunk, b.dlambda_T,
                           b.Gout, b.dlambda0, s.BH, nl, 0);
        return hipGetLastError();
    }
    return s.qkv_bf16 ? bwd_gain_e<bf16_t>(s, b, st) : bwd_gain_e<float>(s, b, st);
}

}  // namespace kdn
