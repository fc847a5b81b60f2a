// kdn_chunk.hip -- chunkwise memory write and read-out of the KDN layer.
//
// The memory recurrence S_t = a_t S_{t-1} + (v_t - a_t S_{t-1} k_t) w_t^T,
// o_t = S_t q_t is a generalised delta rule whose write key w_t is the Kalman
// gain ("Kalman Delta Networks", English abstract: the gain sets how much of
// each token's residual is written; ai-feeds.com summary, section 方法 step 3:
// the write is computed chunk by chunk, as in hardware-friendly delta-rule
// kernels).  Within a chunk of C tokens that
// starts from S0, with local cumulative decay gamma_t = prod_{s<=t} a_s,
// g = log gamma and Gamma_ts = exp(g_t - g_s):
//   A  = strict_tril(K W^T * Gamma),  T = (I + A)^{-1}
//   U  = T (V - diag(gamma) K S0^T)                     (the innovations)
//   O  = diag(gamma) Q S0^T + (tril(Q W^T) * Gamma) U   (diagonal included)
//   S_end = gamma_C S0 + U^T diag(gamma_C / gamma_s) W
// Everything except the S0 terms is local to the chunk.
//
// Two kernels:
//   prep_kernel   two chunks per workgroup, all chunks in parallel: optionally
//                 the gain w from the chunk-boundary precision, then A and the
//                 unit-lower-triangular inverse T (16x16 diagonal blocks by
//                 forward substitution, off-diagonal blocks by block columns
//                 on MFMA), in fp32 or fp32-accurate arithmetic; T is stored
//                 in the input dtype.
//   state_kernel  one workgroup per (head, d_v tile), sequential over chunks:
//                 the S0-dependent products on MFMA (bf16 inputs: 16x16x32
//                 bf16 MFMA with fp32 accumulation; fp32 inputs: 16x16x4 fp32
//                 MFMA).  The fp32 state lives in MFMA accumulators for the
//                 whole sequence; an input-dtype copy of it is kept in LDS as
//                 the operand of the next chunk.
// Operand arrays in LDS are row-major with the contraction index contiguous,
// so every MFMA fragment is one 16-byte (bf16) or 4-byte (fp32) LDS read;
// operands needed with the contraction index strided (W in the state update,
// the token-major R) are read with transposing LDS reads.
#include <algorithm>
#include <cmath>

#include "kdn_device.h"
#include "kdn_launch.h"
#include "kdn_tiles.h"

namespace kdn {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsLimit = 160 * 1024;

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

// index of the off-diagonal block (i, j), i > j, in a packed strictly lower
// block triangle
__device__ __forceinline__ int tri_index(int i, int j) { return i * (i - 1) / 2 + j; }

// 16x16 fp32 blocks of the solve, stored [n][k] with a padded row
constexpr int kBld = 20, kBlk = 16 * kBld;

// acc += A Bt^T for 16x16 blocks: A row-major [m][k] (row stride lda), Bt
// stored [n][k] (row stride kBld).  Each lane reads one 16-byte piece of each;
// the four 16x16x4 fp32 MFMA steps take the contraction in the order
// k = 4 (lane / 16) + step on both operands, which covers every k once.
__device__ __forceinline__ floatx4 mma16_f32(floatx4 acc, const float* A, int lda,
                                             const float* Bt, int lane) {
    const float4 a4 = *reinterpret_cast<const float4*>(A + (lane & 15) * lda + 4 * (lane >> 4));
    const float4 b4 = *reinterpret_cast<const float4*>(Bt + (lane & 15) * kBld + 4 * (lane >> 4));
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, b4.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, b4.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, b4.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, b4.w, acc, 0, 0, 0);
    return acc;
}

// four floats split as hi + lo, both bfloat16 (hi rounded to nearest, lo the
// rounded remainder), packed as 16x16x16 MFMA operands: products of splits
// dropping lo * lo are exact to about 2^-17 relative
struct Bf16Split {
    short4x hi, lo;
};
__device__ __forceinline__ Bf16Split split_bf16(float a, float b, float c, float d) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const uint32_t h01 = pack_bf16(a, b), h23 = pack_bf16(c, d);
    const uint32_t l01 = pack_bf16(a - __uint_as_float(h01 << 16),
                                   b - __uint_as_float(h01 & 0xFFFF0000u));
    const uint32_t l23 = pack_bf16(c - __uint_as_float(h23 << 16),
                                   d - __uint_as_float(h23 & 0xFFFF0000u));
    return Bf16Split{__builtin_bit_cast(short4x, u32x2_t{h01, h23}),
                     __builtin_bit_cast(short4x, u32x2_t{l01, l23})};
}
// acc + X Y for 16x16 blocks given X's operand piece (lane l: row l % 16, k
// 4 (l / 16) .. + 3) and Y split; three bf16 MFMAs
__device__ __forceinline__ floatx4 mma16_split(floatx4 acc, const float4& x, const Bf16Split& y) {
    const Bf16Split xs = split_bf16(x.x, x.y, x.z, x.w);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xs.hi, y.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xs.lo, y.hi, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xs.hi, y.lo, acc, 0, 0, 0);
    return acc;
}

// a 16x16 MFMA result (lane l: rows 4 (l / 16) + e, column l % 16) stored
// transposed, [n][m], one 16-byte store per lane
__device__ __forceinline__ void store_ct(float* dst, floatx4 v, int lane) {
    *reinterpret_cast<float4*>(dst + (lane & 15) * kBld + 4 * (lane >> 4)) =
        make_float4(v[0], v[1], v[2], v[3]);
}

// LDS of the prep kernel: two regions reused as the chunk proceeds.
//   region 1: K [C][LDK] (input dtype), then A with the diagonal blocks of T
//             [C][LDA] (fp32)
//   region 2: W [C][LDK] (input dtype), then the blocks of the solve
//             (fp32)
template <typename E, int DK, int C> struct PrepLds {
    // rows padded by 32 bytes (a stride of 8 mod 16 dwords: conflict-free MFMA
    // fragment reads)
    static constexpr int PAD = 32 / (int)sizeof(E);
    static constexpr int LDK = DK + PAD, LDA = C + 8;
    static constexpr int NT = C / 16;  // 16-token sub-blocks = waves of the gain pass
    static constexpr int NPL = DK >= 64 ? DK / 64 : 1;  // key dims per lane (gain pass)
    static constexpr int R1 = cmax(C * LDK * (int)sizeof(E), C * LDA * 4);
    // region 2 also holds the blocks of T (off-diagonal, and the diagonal ones
    // transposed) while T is formed
    static constexpr int R2 =
        cmax(C * LDK * (int)sizeof(E), (NT * (NT - 1) / 2 + NT) * kBlk * 4);
    static constexpr int BYTES = R1 + R2 + 2 * C * (int)sizeof(float);
    // 16-byte pieces of one chunk's K per thread
    static constexpr int NV = C * DK / Vec16<E>::N;
    static constexpr int IT = (NV + kThreads - 1) / kThreads;
};

// ------------------------------------------------------------ prep kernel
// One workgroup (4 waves) per chunk.
//   gain (fuse_gain), diagonal: wave w takes the 16-token sub-block w and each
//     lane NPL key dimensions.  (1) Wave w > 0 carries the chunk-boundary
//     precision through the scan's prefix product of the chunk's first 16 w
//     tokens to its own start; (2) it walks its 16 tokens (predictive
//     precision, P^- k); (3) the per-token sums k^T P^- k come from a
//     transposing butterfly inside 16-lane groups and two cross-group
//     exchanges; (4) w = P^- k / (k^T P^- k + r) is written by rows.
//     Isotropic: |k|^2 per token, one scalar chain, w = k / (|k|^2 + r lambda^-).
//   A = strict_tril(K W^T * Gamma) on MFMA and T = (I + A)^{-1}: 16x16
//     diagonal blocks in place by forward substitution in fp32 (one lane per
//     column, all blocks in one wave), then block columns T_ij = -T_ii
//     sum_{m=j}^{i-1} A_im T_mj on MFMA, one wave per block column (fp32
//     MFMA for fp32 inputs; for bf16 inputs three bf16 MFMAs per product on
//     hi / lo splits, about 2^-17 relative).

// One chunk's inputs, loaded into registers ahead of their use: K rows, the
// gates of token `lane` (in their storage type G, widened only when used, so
// that no wait for the load is forced early), the chunk-boundary precision of
// the lane's key dimensions and (diagonal, waves past the first) the scan's
// prefix product of the tokens before the wave's sub-block.  Rows past the end
// of the sequence load the last valid row and are zeroed when staged.
template <typename E, typename G, int DK, int C> struct PrepIn {
    u32x4 k[PrepLds<E, DK, C>::IT];
    G a, nu, r;
    float lam[PrepLds<E, DK, C>::NPL];
    float4 pre[PrepLds<E, DK, C>::NPL];
};

template <typename E, typename G, int DK, int C, bool FUSE>
__device__ __forceinline__ void prep_fetch(const E* __restrict__ k, const G* __restrict__ a,
                                           const G* __restrict__ nu, const G* __restrict__ r,
                                           bool diag, const float* __restrict__ lam_chunk,
                                           const float4* __restrict__ agg, const Slab& sl,
                                           int c, int tid, PrepIn<E, G, DK, C>& in) {
    using L = PrepLds<E, DK, C>;
    constexpr int V = Vec16<E>::N, VPR = DK / V, NPL = L::NPL;
    const int lane = tid & 63, wave = wave_id();
    const int t0 = c * C, n = min(C, sl.T - t0);
    const size_t row0 = sl.row0 + t0;
#pragma unroll
    for (int x = 0; x < L::IT; ++x) {
        const int e = tid + kThreads * x;
        if (L::NV % kThreads == 0 || e < L::NV) {
            const int t = e / VPR, c0 = (e % VPR) * V;
            in.k[x] = *reinterpret_cast<const u32x4*>(k + (row0 + min(t, n - 1)) * DK + c0);
        }
    }
    const size_t tok = row0 + min(lane, n - 1);
    in.a = a[tok];
    in.nu = from_f<G>(0.f);
    in.r = from_f<G>(1.f);
#pragma unroll
    for (int d = 0; d < NPL; ++d) {
        in.lam[d] = 1.f;
        in.pre[d] = make_float4(1.f, 0.f, 0.f, 1.f);
    }
    if constexpr (FUSE) {
        in.nu = nu[tok];
        in.r = r[tok];
        if (diag) {
            const int i0 = lane * NPL;
            if (wave < L::NT && i0 < DK) {
#pragma unroll
                for (int d = 0; d < NPL; ++d)
                    in.lam[d] = lam_chunk[(sl.l0 + c) * DK + i0 + d];
                if (wave > 0) {
#pragma unroll
                    for (int d = 0; d < NPL; ++d)
                        in.pre[d] = agg[((sl.c0 + c) * L::NT + wave - 1) * DK + i0 + d];
                }
            }
        } else if (wave == 0) {
            in.lam[0] = lam_chunk[sl.l0 + c];
        }
    }
}

// The work of one chunk; LDS as in PrepLds, inputs already in registers.
template <typename E, typename G, int DK, int C, bool FUSE>
__device__ __forceinline__ void prep_chunk(const E* w_in, bool diag, E* w,
                                           E* __restrict__ Tm, float* __restrict__ gout,
                                           float* __restrict__ dinv, const Slab& sl, int c,
                                           const PrepIn<E, G, DK, C>& in,
                                           unsigned char* smem, float* sden, float* sg,
                                           float4* sgt) {
    using L = PrepLds<E, DK, C>;
    constexpr int LDK = L::LDK, LDA = L::LDA, NT = L::NT, NPL = L::NPL;
    constexpr int V = Vec16<E>::N, VPR = DK / V;
    E* sK = reinterpret_cast<E*>(smem);
    float* sAT = reinterpret_cast<float*>(smem);  // after A is formed
    E* sW = reinterpret_cast<E*>(smem + L::R1);
    float* sZ = reinterpret_cast<float*>(smem + L::R1);  // after A is formed

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int t0 = c * C, n = min(C, sl.T - t0);
    const size_t row0 = sl.row0 + t0;

    // stage K; rows past the end of the sequence are zero (a full chunk, the
    // common case, stores without selects).  A given W (no fused gain: a stage
    // call, not the forward) is read here directly.
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const bool full = n == C;
#pragma unroll
    for (int x = 0; x < L::IT; ++x) {
        const int e = tid + kThreads * x;
        if (L::NV % kThreads == 0 || e < L::NV) {
            const int t = e / VPR, c0 = (e % VPR) * V;
            *reinterpret_cast<u32x4*>(sK + t * LDK + c0) = (full || t < n) ? in.k[x] : zero;
        }
    }
    if constexpr (!FUSE) stage_rows<E, C, DK>(sW, LDK, w_in + row0 * DK, DK, n);
    // lane t of every wave: the gates of token t (padding: a = 1, nu = 0, r = 1)
    float ga = 1.f, ga2 = 1.f, gnu = 0.f, gr = 1.f, gir = 1.f;
    if (lane < n) {
        ga = to_f<G>(in.a);
        ga2 = ga * ga;
        gnu = to_f<G>(in.nu);
        gr = to_f<G>(in.r);
        gir = rcp(gr);
    }
    if (wave == 0) {
        const float g = wave_incl_sum(lane < C ? log2_hw(ga) : 0.f);
        if (lane < C) {
            sg[lane] = g;
            sgt[lane] = make_float4(ga2, gnu, gir, gr);  // read by every lane, token by token
            gout[(sl.c0 + c) * C + lane] = g;  // for the state pass
        }
    }
    sync_lds();

    if constexpr (FUSE) {
        if (diag) {
            const int i0 = lane * NPL, tb0 = 16 * wave;
            const bool act = wave < NT && i0 < DK;
            float kc[16][NPL];
            if (act) {
#pragma unroll
                for (int j = 0; j < 16; ++j) load_dims<E, NPL>(sK + (tb0 + j) * LDK + i0, kc[j]);
            }
            float pk[16][NPL];
            float den = 0.f;
            if (act) {
                // (1) precision at the sub-block start: the chunk-boundary value
                // through the scan's prefix product of the tokens before it
                float lam[NPL];
#pragma unroll
                for (int d = 0; d < NPL; ++d) {
                    const float4 p = in.pre[d];  // the identity on wave 0
                    lam[d] = fmaf(p.x, in.lam[d], p.y) * rcp(fmaf(p.z, in.lam[d], p.w));
                }
                // (2) walk in variance form, P = 1 / lambda: P^- = a^2 P + nu, then
                // P = P^- / (1 + b P^-) (one reciprocal per token); P^- k per token
                float pv[NPL];
#pragma unroll
                for (int d = 0; d < NPL; ++d) pv[d] = rcp(lam[d]);
                float v[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float4 gv = sgt[tb0 + j];
                    const float a2 = gv.x, nut = gv.y, ir = gv.z;
                    v[j] = 0.f;
#pragma unroll
                    for (int d = 0; d < NPL; ++d) {
                        const float kv = kc[j][d];
                        const float pm = fmaf(a2, pv[d], nut);
                        pk[j][d] = kv * pm;
                        const float kpk = kv * pk[j][d];  // k_i^2 P^-_i
                        v[j] += kpk;
                        pv[d] = pm * rcp(fmaf(kpk, ir, 1.f));
                    }
                }
                // (3) k^T P^- k of token tb0 + (lane % 16), summed over all lanes
                den = transpose_sum16(v, lane);
            }
            den += __shfl_xor(den, 16, kWave);
            den += __shfl_xor(den, 32, kWave);
            // lane l: r of token tb0 + l % 16, gathered from the lane that loaded it
            // with every lane active (with d_k < 64 the lanes past d_k are off
            // inside the branch below, and a shuffle reads nothing from them)
            const float rt = __shfl(gr, tb0 + (lane & 15), kWave);
            if (act) {
                const float rden = rcp(den + rt);
                if (dinv && lane < 16 && tb0 + lane < n) dinv[row0 + tb0 + lane] = rden;
                // (4) w rows: converted once, stored to LDS and to HBM (a full
                // chunk with one base address and constant row offsets)
                E out[16][NPL];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float rd = lane_value(rden, j);
#pragma unroll
                    for (int d = 0; d < NPL; ++d) out[j][d] = from_f<E>(pk[j][d] * rd);
                    store_dims<E, NPL>(sW + (tb0 + j) * LDK + i0, out[j]);
                }
                E* wrow = w + (row0 + tb0) * DK + i0;
                if (full) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) store_dims<E, NPL>(wrow + j * DK, out[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        if (tb0 + j < n) store_dims<E, NPL>(wrow + j * DK, out[j]);
                }
            }
        } else {
            // |k|^2 per token (four lanes per token), then one scalar chain
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
                // the chunk's precision walk as an inclusive prefix product of the
                // tokens' Moebius maps (later tokens on the left; padded tokens are
                // the identity), then each token's predictive precision from the
                // posterior after the token before it
                const float kk = lane < C ? sden[lane] : 0.f;
                const float bt = kk * gir * (1.f / static_cast<float>(DK));
                M2 P = {1.f + bt * gnu, bt * ga2, gnu, ga2};
#pragma unroll
                for (int off = 1; off < kWave; off <<= 1) {
                    const M2 o = {__shfl_up(P.a, off, kWave), __shfl_up(P.b, off, kWave),
                                  __shfl_up(P.c, off, kWave), __shfl_up(P.d, off, kWave)};
                    if (lane >= off) P = mob_renorm(mob_mul(P, o));
                }
                const float lam_incl = mob_apply(P, in.lam[0]);
                float lam = __shfl_up(lam_incl, 1, kWave);
                if (lane == 0) lam = in.lam[0];
                const float lm = lam * rcp(fmaf(gnu, lam, ga2));
                if (lane < C) sden[lane] = 1.f / (kk + gr * lm);
            }
            sync_lds();
            constexpr int VPR = DK / V;
            for (int e = tid; e < C * VPR; e += kThreads) {
                const int t = e / VPR, i0 = (e % VPR) * V;
                E out[V];
                const float dn = sden[t];
#pragma unroll
                for (int j = 0; j < V; ++j) out[j] = from_f<E>(to_f<E>(sK[t * LDK + i0 + j]) * dn);
                const uint4 u = *reinterpret_cast<const uint4*>(out);
                *reinterpret_cast<uint4*>(sW + t * LDK + i0) = u;
                if (t < n) *reinterpret_cast<uint4*>(w + (row0 + t) * DK + i0) = u;
            }
        }
    }
    sync_lds();

    // A = strict_tril(K W^T * Gamma) in fp32 (zero on and above the diagonal):
    // the NT (NT + 1) / 2 lower tiles dealt round-robin to the waves, computed
    // into registers, written over K after a barrier
    constexpr int NTILE = NT * (NT + 1) / 2, TPW = (NTILE + 3) / 4;
    floatx4 at[TPW];
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int id = wave + 4 * x;
        int tb = 0, sb = id;
        while (sb > tb) {
            sb -= tb + 1;
            ++tb;
        }
        // the transposed tile W K^T: lane l holds 4 consecutive columns of row
        // 16 tb + l % 16 of A, written with one 16-byte store
        at[x] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (id < NTILE) at[x] = mma_tile<E>(at[x], sW, LDK, 16 * sb, sK, LDK, 16 * tb, 0, DK, lane);
    }
    sync_lds();
    // (the blocks above the diagonal are never read: neither the solve nor the
    // store of T touches them)
#pragma unroll
    for (int x = 0; x < TPW; ++x) {
        const int id = wave + 4 * x;
        if (id < NTILE) {
            int tb = 0, sb = id;
            while (sb > tb) {
                sb -= tb + 1;
                ++tb;
            }
            const int t = 16 * tb + c_col(lane), s0 = 16 * sb + c_row(lane, 0);
            const float gt = sg[t];
            const float4 gs = *reinterpret_cast<const float4*>(sg + s0);
            const floatx4 v = at[x];
            *reinterpret_cast<float4*>(sAT + t * LDA + s0) =
                make_float4((s0 + 0 < t) ? exp2_hw(gt - gs.x) * v[0] : 0.f,
                            (s0 + 1 < t) ? exp2_hw(gt - gs.y) * v[1] : 0.f,
                            (s0 + 2 < t) ? exp2_hw(gt - gs.z) * v[2] : 0.f,
                            (s0 + 3 < t) ? exp2_hw(gt - gs.w) * v[3] : 0.f);
        }
    }
    sync_lds();

    // diagonal 16x16 blocks, in place, all in one wave: forward substitution with
    // lane 16 b + j on column j of block b (row t of A is read before row t of T
    // is written)
    float* sTo = sZ;                                      // [NT (NT - 1) / 2] blocks
    float* sTd = sZ + kBlk * (NT * (NT - 1) / 2);          // [NT] blocks
    if (wave == 0 && (lane >> 4) < NT) {
        const int b0 = 16 * (lane >> 4), col = lane & 15;
        float x[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float arow[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 a4 = *reinterpret_cast<const float4*>(sAT + (b0 + t) * LDA + b0 + 4 * q);
                arow[4 * q] = a4.x;
                arow[4 * q + 1] = a4.y;
                arow[4 * q + 2] = a4.z;
                arow[4 * q + 3] = a4.w;
            }
            float acc = (t == col) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < t; ++s) acc -= arow[s] * x[s];
            x[t] = acc;
            sAT[(b0 + t) * LDA + b0 + col] = acc;
        }
        // T_bb^T (column col of T_bb as a row), the operand layout of the solve
        float* dst = sTd + kBlk * (lane >> 4) + col * kBld;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(dst + 4 * q) =
                make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
    }
    sync_lds();
    // off-diagonal blocks by block columns: wave j forms T_ij for i = j+1, j+2, ...
    // in order, T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj.  A 16x16 MFMA result
    // (lane l: rows 4 (l / 16) + e of column l % 16) is, lane for lane, the B
    // operand of the next product (its contraction index 4 (l / 16) + e), so the
    // column's blocks T_mj stay in registers and the chain has no LDS round
    // trip.  A and the diagonal inverses are read from LDS (A row-major in
    // place, T_jj transposed in its own block); the T_ij are stored transposed,
    // [n][k], for the output below.  bf16 inputs (T is stored in bf16): each
    // 16x16x16 product as three bf16 MFMAs on hi / lo splits, about 2^-17
    // relative, a quarter of the issue time of four fp32 16x16x4 steps; fp32
    // inputs: fp32 MFMA, the steps over two accumulators.
    if (wave < NT - 1) {
        const int j = wave;
        const int r = lane & 15, k4 = 4 * (lane >> 4);
        const float4 d4 =
            *reinterpret_cast<const float4*>(sTd + kBlk * j + r * kBld + k4);  // T_jj as B
        if constexpr (sizeof(E) == 2) {
            Bf16Split tc[NT];  // T_mj split, m = j .. i - 1
#pragma unroll
            for (int m = 0; m < NT; ++m) tc[m] = split_bf16(d4.x, d4.y, d4.z, d4.w);
#pragma unroll
            for (int i = 1; i < NT; ++i) {
                if (i <= j) continue;
                floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NT - 1; ++m) {
                    if (m < j || m >= i) continue;
                    z = mma16_split(
                        z, *reinterpret_cast<const float4*>(sAT + (16 * i + r) * LDA + 16 * m + k4),
                        tc[m]);
                }
                const floatx4 t = mma16_split(
                    floatx4{0.f, 0.f, 0.f, 0.f},
                    *reinterpret_cast<const float4*>(sAT + (16 * i + r) * LDA + 16 * i + k4),
                    split_bf16(z[0], z[1], z[2], z[3]));
                const floatx4 tij = -t;
#pragma unroll
                for (int m = 1; m < NT; ++m)
                    if (m == i) tc[m] = split_bf16(tij[0], tij[1], tij[2], tij[3]);
                store_ct(sTo + kBlk * tri_index(i, j), tij, lane);
            }
        } else {
            floatx4 tc[NT];  // T_mj in the MFMA result layout, m = j .. i - 1
#pragma unroll
            for (int m = 0; m < NT; ++m) tc[m] = floatx4{d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int i = 1; i < NT; ++i) {
                if (i <= j) continue;
                floatx4 za = {0.f, 0.f, 0.f, 0.f}, zb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int m = 0; m < NT - 1; ++m) {
                    if (m < j || m >= i) continue;
                    const float4 a4 =
                        *reinterpret_cast<const float4*>(sAT + (16 * i + r) * LDA + 16 * m + k4);
                    za = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, tc[m][0], za, 0, 0, 0);
                    zb = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, tc[m][2], zb, 0, 0, 0);
                    za = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, tc[m][1], za, 0, 0, 0);
                    zb = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, tc[m][3], zb, 0, 0, 0);
                }
                const floatx4 z = za + zb;
                const float4 t4 =
                    *reinterpret_cast<const float4*>(sAT + (16 * i + r) * LDA + 16 * i + k4);
                floatx4 ta = {0.f, 0.f, 0.f, 0.f}, tb = {0.f, 0.f, 0.f, 0.f};
                ta = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.x, z[0], ta, 0, 0, 0);
                tb = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.z, z[2], tb, 0, 0, 0);
                ta = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.y, z[1], ta, 0, 0, 0);
                tb = __builtin_amdgcn_mfma_f32_16x16x4f32(t4.w, z[3], tb, 0, 0, 0);
                const floatx4 tij = -(ta + tb);
#pragma unroll
                for (int m = 1; m < NT; ++m)
                    if (m == i) tc[m] = tij;
                store_ct(sTo + kBlk * tri_index(i, j), tij, lane);
            }
        }
    }
    sync_lds();
    E* Tout = Tm + (sl.c0 + c) * (size_t)(C * C);
    for (int e = tid; e < C * C / V; e += kThreads) {
        const int t = e / (C / V), s0 = (e % (C / V)) * V;
        const int tb = t >> 4, sb = s0 >> 4;
        E out[V];
        if (sb == tb) {
#pragma unroll
            for (int j = 0; j < V; ++j) out[j] = from_f<E>(sAT[t * LDA + s0 + j]);
        } else if (sb < tb) {  // stored transposed
            const float* src = sTo + kBlk * tri_index(tb, sb) + (s0 & 15) * kBld + (t & 15);
#pragma unroll
            for (int j = 0; j < V; ++j) out[j] = from_f<E>(src[j * kBld]);
        } else {
#pragma unroll
            for (int j = 0; j < V; ++j) out[j] = from_f<E>(0.f);
        }
        *reinterpret_cast<uint4*>(Tout + t * C + s0) = *reinterpret_cast<const uint4*>(out);
    }
}

// Two chunks per workgroup (2 blockIdx.x and the next): the second chunk's
// inputs are loaded at the start and arrive while the first is processed.
// VL: a packed batch (blockIdx.y = sequence * H + head); workgroups past the
// sequence's chunks return at once.
template <typename E, typename G, int DK, int C, bool FUSE, bool VL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void prep_kernel(
    const E* __restrict__ k, const G* __restrict__ a, const G* __restrict__ nu,
    const G* __restrict__ r, bool diag, const float* __restrict__ lam_chunk,
    const float4* __restrict__ agg, E* __restrict__ w, E* __restrict__ Tm,
    float* __restrict__ gout, float* __restrict__ dinv, int T, int NC, Packed pk) {
    using L = PrepLds<E, DK, C>;
    __shared__ __align__(16) unsigned char smem[L::R1 + L::R2];
    __shared__ __align__(16) float sden[C];
    __shared__ __align__(16) float sg[C];
    __shared__ float4 sgt[C];  // per token: a^2, nu, 1/r, r
    const int tid = threadIdx.x;
    const Slab sl = slab_of<VL>(blockIdx.y, T, NC, pk);
    const int c0 = 2 * blockIdx.x, c1 = c0 + 1;
    if (VL && c0 >= sl.nc) return;
    PrepIn<E, G, DK, C> in0, in1;
    prep_fetch<E, G, DK, C, FUSE>(k, a, nu, r, diag, lam_chunk, agg, sl, c0, tid, in0);
    prep_fetch<E, G, DK, C, FUSE>(k, a, nu, r, diag, lam_chunk, agg, sl, min(c1, sl.nc - 1), tid,
                                  in1);
    prep_chunk<E, G, DK, C, FUSE>(w, diag, w, Tm, gout, dinv, sl, c0, in0, smem, sden, sg, sgt);
    if (c1 < sl.nc) {
        sync_lds();  // the second chunk's staging overwrites K / A / T
        prep_chunk<E, G, DK, C, FUSE>(w, diag, w, Tm, gout, dinv, sl, c1, in1, smem, sden, sg,
                                      sgt);
    }
}

// ----------------------------------------------------------- state kernel
// One workgroup of 8 waves per (head, d_v tile), sequential over the chunks.
// Per chunk, with S the state at the chunk start and gamma_t = 2^(g_t):
//   phase A  every wave, one (2 j-tiles x 1 t-tile) block:
//              X^T = S K^T  ->  R = V - diag(gamma) X   (stored token-major)
//              Y   = diag(gamma) Q S^T, kept as the O^T accumulator
//            (both products share the S fragments); in the layer shape (four
//            t-tiles and j-tiles, eight waves) also M = tril(Q W^T) * Gamma
//   phase B  U = T R (stored as U^T, and as U^T scaled by gamma_C / gamma_t);
//            in the layer shape on all waves, which then stage the next
//            chunk's K, Q, V and W (the first three were last read in phase A,
//            W goes to the other of two buffers); otherwise U on waves 0-3 and
//            M on waves 4-7
//   phase C  every wave: O^T += U^T M^T for its block, written out; and one
//            block of the state update S^T <- gamma_C S^T + W^T diag(gamma_C/gamma_t) U;
//            then the rest of the next chunk (loaded from HBM into one of two
//            register sets during the previous chunk) is written to LDS with its
//            decay tables, and the new state as the next operand.  The chunk
//            after next is loaded into the other register set meanwhile, in
//            three parts at the starts of the three phases.
// Operands stored with the contraction index strided (token-major R and W) are
// read with transposing LDS reads (ds_read_b64_tr_b16).  Barriers are LDS-only
// (sync_lds) so that the next chunk's global loads stay in flight across them.
// Decays use base-2 logarithms: g_t = sum_{s<=t} log2 a_s, Gamma_ts = 2^(g_t-g_s).
// t-tile of a phase-A / output job: odd groups of NT jobs run the t-tiles in
// reverse, so that the two waves sharing a SIMD (w and w + 4) get output
// contractions of complementary depth
template <int NT> __device__ __forceinline__ int a_tile(int job) {
    return ((job / NT) & 1) ? NT - 1 - job % NT : job % NT;
}

// LDS of the state kernel
template <typename E, int DK, int DVT, int C> struct StateLds {
    using G = StateCfg<E, DK, DVT, C>;
    E K[C * G::LDK];
    E W[2][C * G::LDK];  // double-buffered: read by the state update
    E Q[C * G::LDK];
    E S[DVT * G::LDK];   // state tile S[j][i] as an operand
    E R[C * G::LDV];     // R [t][j]
    E U[DVT * G::LDC];   // U^T [j][t]
    E Us[DVT * G::LDC];  // U^T scaled by gamma_C / gamma_t
    E Tt[C * G::LDC];    // (I + A)^{-1}  [t][s]
    E M[C * G::LDC];     // tril(Q W^T) * Gamma  [t][s]
    E V[C * G::LDV];
    float g[2][C];       // g_t (base 2)
    float gam[2][C];     // gamma_t = 2^g_t
    float del[2][C];     // gamma_C / gamma_t
    // (two sets of decay tables, used by alternate chunks when the M tiles of
    // the next chunk are formed ahead; set 0 only otherwise)
};

// The layer shape with a read-out (four t-tiles, four j-tiles, eight waves):
// the M tiles of chunk c + 1 are formed in phase C of chunk c, into the
// buffer that held chunk c's R, so that phase A holds the two contractions of
// the state alone; R and M trade buffers from chunk to chunk, and the decay
// tables of chunk c + 1 go to the other table set in phase B.
#ifndef KDN_M_AHEAD
#define KDN_M_AHEAD 1
#endif
template <typename E, int DK, int DVT, int C, bool OUT>
constexpr bool state_m_ahead() {
    using G = StateCfg<E, DK, DVT, C>;
    return KDN_M_AHEAD && OUT && G::NT == 4 && G::NV == 4 && G::BT == 2 && G::BV == 2 &&
           G::NW == 8;
}

// The ten lower 16 x 16 tiles of M = tril(Q W^T) * Gamma at the layer shape,
// each formed transposed (W Q^T, full depth), masked and scaled, and stored as
// M[t][s] (element e <-> s = 16 ss + 4 (lane/16) + e, t = 16 tt + lane % 16):
// waves 0-3 two tiles that share their W fragments, (0,0)+(0,1), (0,2)+(0,3),
// (1,1)+(1,2), (2,2)+(2,3); waves 4 and 5 one tile, (1,3) and (3,3).
template <typename E, int DK, int LDK, int LDC>
__device__ __forceinline__ void state_m_tiles(E* sM, const E* sW, const E* sQ, const float* g,
                                              int wave, int lane) {
    auto m_store = [&](int ss, int tt, floatx4 mv) __attribute__((always_inline)) {
        const int s0 = 16 * ss + 4 * (lane >> 4);
        const int t = 16 * tt + (lane & 15);
        const float gt = g[t];
        const float4 gs = *reinterpret_cast<const float4*>(g + s0);
        store4<E>(sM + t * LDC + s0, (s0 + 0 <= t) ? exp2_hw(gt - gs.x) * mv[0] : 0.f,
                  (s0 + 1 <= t) ? exp2_hw(gt - gs.y) * mv[1] : 0.f,
                  (s0 + 2 <= t) ? exp2_hw(gt - gs.z) * mv[2] : 0.f,
                  (s0 + 3 <= t) ? exp2_hw(gt - gs.w) * mv[3] : 0.f);
    };
    if (wave < 4) {
        const int ss = wave < 2 ? 0 : wave - 1, tt = wave == 1 ? 2 : ss;
        floatx4 m[1][2] = {{floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}}};
        mma_block<E, 1, 2>(m, sW, LDK, 16 * ss, sQ, LDK, 16 * tt, 0, DK, lane);
        m_store(ss, tt, m[0][0]);
        m_store(ss, tt + 1, m[0][1]);
    } else if (wave < 6) {
        const int ss = wave == 4 ? 1 : 3;
        m_store(ss, 3, mma_tile<E>(floatx4{0.f, 0.f, 0.f, 0.f}, sW, LDK, 16 * ss, sQ, LDK, 48, 0,
                                   DK, lane));
    }
}

// A state pass over sequence segments (kernel argument): each head's chunks
// cut into nseg runs, the first of L0 chunks and the others of Lc (the last
// may be shorter); this launch runs segments g0 .. g0 + nsegL - 1 of every
// head, each with ntv value-row tiles and nta identity-row tiles.
constexpr int kStateCUs = 256;  // compute units: one state workgroup each

struct SegPlan {
    int nseg = 1, Lc = 0, L0 = 0, g0 = 0, nsegL = 1, ntv = 1, nta = 0;
    int map_wgs = 0, map_jobs = 0;  // maps launch: workgroups running maps, jobs per workgroup
    float* Sseg = nullptr;        // [BH][nseg][DV][DK]: start state of each segment
    float* Aseg = nullptr;        // [BH][nseg][DK][DK]: linear part of each segment's map
};

// what every wave of a state workgroup knows about its problem
template <typename E> struct StateArgs {
    const E *q, *k, *v, *w, *Tm;
    const float* gin;
    E* o;
    Slab sl;  // the rows and chunks of the head (or of one segment of it)
    int j0, DV, tid, lane, wave;
    int jv;       // first column of V read for this tile (j0, or 0 for identity rows)
    bool zero_v;  // identity rows of a segment map: V is zero
};

// One chunk c of the state pass.  LDS holds chunk c on entry.  The register
// set (lk..lg) has been staged already and now receives chunk c + 2 from HBM;
// the set (nk..ng) holds chunk c + 1 and is staged into LDS in phase C.
// OUT = false: no read-out (Y, M and O are not formed, Q is not loaded).
template <typename E, int DK, int DVT, int C, bool OUT>
__device__ __forceinline__ void state_chunk(
    const StateArgs<E>& A, StateLds<E, DK, DVT, C>& L, StateAcc<E, DK, DVT, C>& accS, int c,
    u32x4 (&lk)[StateCfg<E, DK, DVT, C>::PK], u32x4 (&lq)[StateCfg<E, DK, DVT, C>::PK],
    u32x4 (&lw)[StateCfg<E, DK, DVT, C>::PK], u32x4 (&lv)[StateCfg<E, DK, DVT, C>::PV],
    u32x4 (&lt)[StateCfg<E, DK, DVT, C>::PT], float& lg,
    const u32x4 (&nk)[StateCfg<E, DK, DVT, C>::PK], const u32x4 (&nq)[StateCfg<E, DK, DVT, C>::PK],
    const u32x4 (&nw)[StateCfg<E, DK, DVT, C>::PK], const u32x4 (&nv)[StateCfg<E, DK, DVT, C>::PV],
    const u32x4 (&nt)[StateCfg<E, DK, DVT, C>::PT], float ng) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int LDK = G::LDK, LDC = G::LDC, LDV = G::LDV;
    constexpr int BT = G::BT, BV = G::BV, BI = G::BI, BVA = G::BVA;
    constexpr int NVB = G::NVB, NT = G::NT;
    const int lane = A.lane, wave = A.wave;
    const int t0 = c * C, n = min(C, A.sl.T - t0);
    const size_t row0 = A.sl.row0 + t0;
    E* sWc = L.W[c & 1];
    __builtin_amdgcn_sched_barrier(0);
    state_prefetch<E, DK, DVT, C, kLoadKQ, OUT>(A.q, A.k, A.v, A.w, A.Tm, A.gin, A.sl, A.jv, A.DV,
                                           c + 2, A.tid, lane, lk, lq, lw, lv, lt, lg);
    __builtin_amdgcn_sched_barrier(0);  // keep the three load bursts apart

    // the layer shape (four t-tiles, four j-tiles, eight waves): M is formed in
    // phase A, where the first wave of each SIMD has slack, or (kAhead, with a
    // read-out) in phase C of the chunk before; U = T R takes all eight waves in
    // phase B
    constexpr bool kMInA = NT == 4 && G::NV == 4 && BT == 2 && BV == 2 && G::NW == 8;
    constexpr bool kAhead = state_m_ahead<E, DK, DVT, C, OUT>();
    static_assert(!kAhead || (kMInA && LDV == LDC), "R and M trade buffers");
    // this chunk's decay tables and the next chunk's; its R and M buffers
    const int tc = kAhead ? (c & 1) : 0, tn = kAhead ? ((c + 1) & 1) : 0;
    const float* gT = L.g[tc];
    const float* gamT = L.gam[tc];
    const float* delT = L.del[tc];
    E* const Rb = kAhead && (c & 1) ? L.M : L.R;
    E* const Mb = kAhead && (c & 1) ? L.R : L.M;

    // ---------------- phase A: X^T = S K^T -> R ;  Y = S Q^T
    // block (jb: BVA j-tiles, tb: one t-tile); C-layout element e <->
    // j = 16 (jb + bv) + 4 (lane/16) + e, t = 16 tb + lane % 16
    floatx4 accY[G::APW][BVA][1];
#pragma unroll
    for (int x = 0; x < G::APW; ++x) {
        const int job = wave + G::NW * x;
        const int jb = (job / NT) * BVA, tb = a_tile<NT>(job);
        floatx4 xt[BVA][1];
#pragma unroll
        for (int bv = 0; bv < BVA; ++bv) {
            xt[bv][0] = floatx4{0.f, 0.f, 0.f, 0.f};
            accY[x][bv][0] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
        if (job < G::NAJ) {
            using M = Mma<E>;
#pragma unroll
            for (int kk = 0; kk < DK; kk += M::KS) {
                typename M::frag_t fs[BVA];
#pragma unroll
                for (int bv = 0; bv < BVA; ++bv)
                    fs[bv] = M::frag(L.S, LDK, 16 * (jb + bv), kk, lane);
                const auto fk = M::frag(L.K, LDK, 16 * tb, kk, lane);
                if constexpr (OUT) {
                    const auto fq = M::frag(L.Q, LDK, 16 * tb, kk, lane);
#pragma unroll
                    for (int bv = 0; bv < BVA; ++bv) {
                        xt[bv][0] = M::mma(fs[bv], fk, xt[bv][0]);
                        accY[x][bv][0] = M::mma(fs[bv], fq, accY[x][bv][0]);
                    }
                } else {
#pragma unroll
                    for (int bv = 0; bv < BVA; ++bv) xt[bv][0] = M::mma(fs[bv], fk, xt[bv][0]);
                }
            }
            const int t = 16 * tb + (lane & 15);
            const float gt = gamT[t];
            static_assert(BVA == 2, "R and V tiles pair along j");
            float vt[BVA][4];
            load8x2<E>(L.V + t * LDV + 16 * jb, L.V + t * LDV + 16 * jb + 16, vt[0], vt[1], lane);
            floatx4 rv[BVA];
#pragma unroll
            for (int bv = 0; bv < BVA; ++bv) {
                const float* vv = vt[bv];
                const floatx4 xv = xt[bv][0];
                rv[bv] = floatx4{vv[0] - gt * xv[0], vv[1] - gt * xv[1], vv[2] - gt * xv[2],
                                 vv[3] - gt * xv[3]};
                if constexpr (OUT) accY[x][bv][0] = accY[x][bv][0] * gt;
            }
            E* row = Rb + t * LDV + 16 * jb;
            store8x2<E>(row, row + 16, rv[0], rv[1], lane);
        }
    }
    if constexpr (kMInA && OUT && !kAhead)
        state_m_tiles<E, DK, LDK, LDC>(L.M, sWc, L.Q, gT, wave, lane);
    sync_lds();
    state_prefetch<E, DK, DVT, C, kLoadW, OUT>(A.q, A.k, A.v, A.w, A.Tm, A.gin, A.sl, A.jv, A.DV,
                                          c + 2, A.tid, lane, lk, lq, lw, lv, lt, lg);
    __builtin_amdgcn_sched_barrier(0);  // keep the three load bursts apart

    // ---------------- phase B
    const float gC = gamT[C - 1];  // read before the tables are restaged
    if constexpr (kMInA) {
        // U = T R (T lower triangular: contract only up to the block's last row):
        // a pair of t-tiles x one j-tile per wave, the deep pair on the first
        // wave of each SIMD; stored as U^T and as U^T scaled by gamma_C / gamma_t
        const int tb = wave < 4 ? 2 : 0, jv = wave & 3;
        floatx4 u[2][1] = {{floatx4{0.f, 0.f, 0.f, 0.f}}, {floatx4{0.f, 0.f, 0.f, 0.f}}};
        mma_block<E, 2, 1, false, true>(u, L.Tt, LDC, 16 * tb, Rb, LDV, 16 * jv, 0,
                                        16 * (tb + 2), lane);
        floatx4 us[2];
#pragma unroll
        for (int bt = 0; bt < 2; ++bt) {
            const int t = 16 * (tb + bt) + 4 * (lane >> 4);
            const float4 d4 = *reinterpret_cast<const float4*>(delT + t);
            const floatx4 uv = u[bt][0];
            us[bt] = floatx4{d4.x * uv[0], d4.y * uv[1], d4.z * uv[2], d4.w * uv[3]};
        }
        const int j = 16 * jv + (lane & 15);
        store8x2<E>(L.U + j * LDC + 16 * tb, L.U + j * LDC + 16 * tb + 16, u[0][0], u[1][0], lane);
        store8x2<E>(L.Us + j * LDC + 16 * tb, L.Us + j * LDC + 16 * tb + 16, us[0], us[1], lane);
        // K, Q, V and W of chunk c + 1 (the first three were last read in phase A;
        // W goes to the other buffer), and with kAhead its decay tables (to the
        // other set): staged here, where the waves have slack
        if (c + 1 < A.sl.nc)
            state_stage<E, DK, DVT, C, kAhead ? (kStageKQWV | kStageTab) : kStageKQWV, OUT>(
                L.K, L.Q, L.W[(c + 1) & 1], L.V, L.Tt, L.g[tn], L.gam[tn], L.del[tn],
                min(C, A.sl.T - (c + 1) * C), A.tid, lane, wave, nk, nq, nw, nv, nt, ng,
                A.zero_v);
    } else if (wave < 4) {
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
                mma_block<E, BT, BV, false, true>(u, L.Tt, LDC, 16 * tb, Rb, LDV, 16 * jb, 0,
                                                  16 * (tb + BT), lane);
                floatx4 us[BT][BV];
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const int t = 16 * (tb + bt) + 4 * (lane >> 4);
                    const float4 d4 = *reinterpret_cast<const float4*>(delT + t);
#pragma unroll
                    for (int bv = 0; bv < BV; ++bv) {
                        const floatx4 uv = u[bt][bv];
                        us[bt][bv] = floatx4{d4.x * uv[0], d4.y * uv[1], d4.z * uv[2], d4.w * uv[3]};
                    }
                }
#pragma unroll
                for (int bv = 0; bv < BV; ++bv) {
                    const int j = 16 * (jb + bv) + (lane & 15);
                    if constexpr (BT == 2) {
                        store8x2<E>(L.U + j * LDC + 16 * tb, L.U + j * LDC + 16 * tb + 16,
                                    u[0][bv], u[1][bv], lane);
                        store8x2<E>(L.Us + j * LDC + 16 * tb, L.Us + j * LDC + 16 * tb + 16,
                                    us[0][bv], us[1][bv], lane);
                    } else {
                        const int t = 16 * tb + 4 * (lane >> 4);
                        const floatx4 uv = u[0][bv], sv = us[0][bv];
                        store4<E>(L.U + j * LDC + t, uv[0], uv[1], uv[2], uv[3]);
                        store4<E>(L.Us + j * LDC + t, sv[0], sv[1], sv[2], sv[3]);
                    }
                }
            }
        }
    }
    if (OUT && !kMInA && wave >= 4) {
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
                mma_block<E, BT, BT>(m, sWc, LDK, 16 * sbb * BT, L.Q, LDK, 16 * tbb * BT, 0, DK,
                                     lane);
#pragma unroll
                for (int bt = 0; bt < BT; ++bt) {
                    const int t = 16 * (tbb * BT + bt) + (lane & 15);
                    const float gt = gT[t];
                    floatx4 mm[BT];
#pragma unroll
                    for (int bs = 0; bs < BT; ++bs) {
                        const int s0 = 16 * (sbb * BT + bs) + 4 * (lane >> 4);
                        const float4 gs = *reinterpret_cast<const float4*>(gT + s0);
                        const floatx4 mv = m[bs][bt];
                        mm[bs] = floatx4{(s0 + 0 <= t) ? exp2_hw(gt - gs.x) * mv[0] : 0.f,
                                         (s0 + 1 <= t) ? exp2_hw(gt - gs.y) * mv[1] : 0.f,
                                         (s0 + 2 <= t) ? exp2_hw(gt - gs.z) * mv[2] : 0.f,
                                         (s0 + 3 <= t) ? exp2_hw(gt - gs.w) * mv[3] : 0.f};
                    }
                    E* row = L.M + t * LDC + 16 * sbb * BT;
                    if constexpr (BT == 2) {
                        store8x2<E>(row, row + 16, mm[0], mm[1], lane);
                    } else {
                        const floatx4 v = mm[0];
                        store4<E>(row + 4 * (lane >> 4), v[0], v[1], v[2], v[3]);
                    }
                }
            }
        }
    }
    sync_lds();
    state_prefetch<E, DK, DVT, C, kLoadVTG, OUT>(A.q, A.k, A.v, A.w, A.Tm, A.gin, A.sl, A.jv, A.DV,
                                            c + 2, A.tid, lane, lk, lq, lw, lv, lt, lg);
    __builtin_amdgcn_sched_barrier(0);  // keep the three load bursts apart

    // ---------------- phase C: O^T += U^T M^T ; state update ; stage chunk c + 1
#pragma unroll
    for (int x = 0; x < G::APW; ++x) {
        const int job = wave + G::NW * x;
        if (OUT && job < G::NAJ) {
            const int jb = (job / NT) * BVA, tb = a_tile<NT>(job);
            mma_block<E, BVA, 1>(accY[x], L.U, LDC, 16 * jb, Mb, LDC, 16 * tb, 0, 16 * (tb + 1),
                                 lane);
            const int t = 16 * tb + (lane & 15);
            E* orow = A.o + (row0 + t) * A.DV + A.j0 + 16 * jb;
            // (o is NULL when the backward recomputes the forward for its states)
            store8x2_if<E>(t < n && A.o, orow, orow + 16, accY[x][0][0], accY[x][1][0], lane);
        }
    }
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
            mma_block<E, BI, BV, true>(accS[x], sWc, LDK, 16 * ib, L.Us, LDC, 16 * jb, 0, C,
                                       lane);
        }
    }
    // kAhead: the M tiles of chunk c + 1 (its Q, W and tables were staged in
    // phase B) into the buffer that held this chunk's R
    if constexpr (kAhead)
        if (c + 1 < A.sl.nc)
            state_m_tiles<E, DK, LDK, LDC>(Rb, L.W[(c + 1) & 1], L.Q, L.g[tn], wave, lane);
    // nothing staged here is read in phase C (W goes to the other buffer)
    if (c + 1 < A.sl.nc)
        state_stage<E, DK, DVT, C, kMInA ? (kAhead ? kStageTm : kStageT) : kStageAll, OUT>(
            L.K, L.Q, L.W[(c + 1) & 1], L.V, L.Tt, L.g[tn], L.gam[tn], L.del[tn],
            min(C, A.sl.T - (c + 1) * C),
            A.tid, lane, wave, nk, nq, nw, nv, nt, ng, A.zero_v);
    state_write<E, DK, DVT, C>(accS, L.S, wave, lane);
    sync_lds();
}

// VL: a packed batch, head = sequence * H + head within the sequence.
// OUT: the read-out o is formed and written.
// SEG: the head's chunks are cut into segments (SegPlan) and each workgroup
//   runs one (head, segment, tile).  With OUT, a segment starts from its true
//   start state (S0, or the start state of segment g in seg.Sseg) and writes
//   o, and the last segment S_T; segment 0 (run by the maps launch) also
//   writes its end state, the start state of segment 1, into seg.Sseg[1].
//   Without OUT it forms the segment's affine map S -> S A_g + B_g: value
//   tiles run segment g from zero (B_g) and write the end state into
//   seg.Sseg[g + 1]; identity tiles (rows of the d_k x d_k identity, V = 0)
//   write A_g into seg.Aseg[g].
template <typename E, int DK, int DVT, int C, bool VL, bool OUT, bool SEG>
__device__ __forceinline__ void state_body(StateLds<E, DK, DVT, C>& L, const E* __restrict__ q,
                                           const E* __restrict__ k, const E* __restrict__ v,
                                           const float* __restrict__ gin,
                                           const E* __restrict__ w, const E* __restrict__ Tm,
                                           const float* S0, E* __restrict__ o, float* S_T,
                                           E* __restrict__ Sc, int T, int DV, int NC, Packed pk,
                                           const SegPlan& seg, int head, int g, int tile) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int BI = G::BI, BV = G::BV, NVB = G::NVB;
    const int tid = threadIdx.x;
    const bool idt = SEG && !OUT && tile >= seg.ntv;  // identity rows of a segment map
    Slab sl = slab_of<VL>(head, T, NC, pk);
    if constexpr (SEG) {
        // segment 0 holds L0 chunks, the others Lc each (the last may be
        // shorter); packed batches cut each sequence into the call's segment
        // count, all of one length (a short sequence's last segments may be
        // empty: identity maps)
        const int Lc = VL ? (sl.nc + seg.nseg - 1) / seg.nseg : seg.Lc;
        const int L0 = VL ? Lc : seg.L0;
        const int cb = g == 0 ? 0 : min(L0 + (g - 1) * Lc, sl.nc);
        const int ce = min(cb + (g == 0 ? L0 : Lc), sl.nc);
        sl.row0 += (size_t)cb * C;
        sl.T = max(0, min(sl.T - cb * C, (ce - cb) * C));
        sl.nc = ce - cb;
        sl.c0 += cb;
    }
    const size_t bh = head;
    const int j0 = (idt ? tile - seg.ntv : tile) * DVT;  // first row of the tile
    // rows of the tile that exist: identity tiles hold the d_k rows of A_g,
    // and with d_k < DVT only the first d_k of their rows
    const int nrows = idt ? min(DVT, DK - j0) : DVT;
    // the tile's start and end state rows (stride DK); NULL start: zero
    const float* Sin = S0 ? S0 + (bh * DV + j0) * DK : nullptr;
    float* Sout = S_T ? S_T + (bh * DV + j0) * DK : nullptr;
    if constexpr (SEG) {
        const size_t slot = bh * seg.nseg + g;
        if constexpr (OUT) {
            if (g > 0) Sin = seg.Sseg + (slot * DV + j0) * DK;
            if (g != seg.nseg - 1) Sout = g == 0 ? seg.Sseg + ((slot + 1) * DV + j0) * DK : nullptr;
        } else if (idt) {
            Sin = nullptr;
            Sout = seg.Aseg + (slot * DK + j0) * DK;
        } else {
            Sin = nullptr;
            Sout = seg.Sseg + ((slot + 1) * DV + j0) * DK;
        }
    }
    const StateArgs<E> A{q,   k,    v,         w,    Tm,       gin,      o, sl, j0, DV, tid,
                         tid & 63, wave_id(), idt ? 0 : j0, idt};
    const int lane = A.lane, wave = A.wave;

    // two register sets receive chunks from HBM two chunks ahead of their use
    u32x4 pkA[G::PK], pqA[G::PK], pwA[G::PK], pvA[G::PV], ptA[G::PT];
    u32x4 pkB[G::PK], pqB[G::PK], pwB[G::PK], pvB[G::PV], ptB[G::PT];
    float pgA = 0.f, pgB = 0.f;

    StateAcc<E, DK, DVT, C> accS;
#pragma unroll
    for (int x = 0; x < G::SPW; ++x) {
        const int job = wave + G::NW * x;
        const int ib = (job / NVB) * BI, jb = (job % NVB) * BV;
#pragma unroll
        for (int bi = 0; bi < BI; ++bi)
#pragma unroll
            for (int bv = 0; bv < BV; ++bv) {
                accS[x][bi][bv] = floatx4{0.f, 0.f, 0.f, 0.f};
                const int i = 16 * (ib + bi) + 4 * (lane >> 4);
                const int j = 16 * (jb + bv) + (lane & 15);
                if (job < G::NSJ && Sin) {
                    const float4 s4 = *reinterpret_cast<const float4*>(Sin + (size_t)j * DK + i);
                    accS[x][bi][bv] = floatx4{s4.x, s4.y, s4.z, s4.w};
                } else if (job < G::NSJ && idt) {
                    const int r = j0 + j;  // identity row r: S[r][i] = (i == r)
                    accS[x][bi][bv] = floatx4{i == r ? 1.f : 0.f, i + 1 == r ? 1.f : 0.f,
                                              i + 2 == r ? 1.f : 0.f, i + 3 == r ? 1.f : 0.f};
                }
            }
    }

    if (sl.nc > 0) {
        state_prefetch<E, DK, DVT, C, kLoadAll, OUT>(q, k, v, w, Tm, gin, sl, A.jv, DV, 0, tid,
                                                     lane, pkA, pqA, pwA, pvA, ptA, pgA);
        state_prefetch<E, DK, DVT, C, kLoadAll, OUT>(q, k, v, w, Tm, gin, sl, A.jv, DV, 1, tid,
                                                     lane, pkB, pqB, pwB, pvB, ptB, pgB);
        state_stage<E, DK, DVT, C, kStageAll, OUT>(L.K, L.Q, L.W[0], L.V, L.Tt, L.g[0],
                                                   L.gam[0], L.del[0], min(C, sl.T), tid, lane,
                                                   wave, pkA, pqA, pwA, pvA, ptA, pgA, idt);
    }
    state_write<E, DK, DVT, C>(accS, L.S, wave, lane);
    sync_lds();
    if constexpr (state_m_ahead<E, DK, DVT, C, OUT>()) {
        // the first chunk's M tiles (later chunks form the next chunk's in phase C)
        if (sl.nc > 0) state_m_tiles<E, DK, G::LDK, G::LDC>(L.M, L.W[0], L.Q, L.g[0], wave, lane);
        sync_lds();
    }

    // the two sets alternate roles from chunk to chunk
    // (Sc: the state at every chunk start, kept for the backward pass)
    for (int c = 0; c < sl.nc; c += 2) {
        if (Sc) state_copy_out<E, DK, DVT, C>(L.S, Sc + ((sl.c0 + c) * DV + j0) * DK, tid);
        state_chunk<E, DK, DVT, C, OUT>(A, L, accS, c, pkA, pqA, pwA, pvA, ptA, pgA, pkB, pqB,
                                        pwB, pvB, ptB, pgB);
        if (c + 1 < sl.nc) {
            if (Sc)
                state_copy_out<E, DK, DVT, C>(L.S, Sc + ((sl.c0 + c + 1) * DV + j0) * DK, tid);
            state_chunk<E, DK, DVT, C, OUT>(A, L, accS, c + 1, pkB, pqB, pwB, pvB, ptB, pgB, pkA,
                                            pqA, pwA, pvA, ptA, pgA);
        }
    }
    if (Sout) {
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
                        if (j < nrows)
                            *reinterpret_cast<float4*>(Sout + (size_t)j * DK + i) =
                                make_float4(sv[0], sv[1], sv[2], sv[3]);
                    }
            }
        }
    }
}

// One workgroup per CU (its LDS footprint) = two waves per SIMD: give each wave
// the full 256-register budget instead of spilling to reach more waves.
// Workgroups go to the 8 XCDs round-robin by linear id: the tiles of one unit
// (a head, or a (segment, head) pair) get ids equal mod 8, so they share one
// XCD's L2 for K, Q, W and T.  Segmented launches number their units segment
// by segment.  The maps launch has at most one workgroup per CU, so that no
// run waits for a CU to come free: its first seg.map_wgs workgroups each form
// seg.map_jobs (segment, head, tile) maps of segments 1 .. nseg - 2 in turn
// (job r of workgroup x is job x + r * map_wgs), the rest run segment 0's
// value tiles with read-out.
template <typename E, int DK, int DVT, int C, bool VL, bool OUT, bool SEG>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(1, 2))) void state_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const float* __restrict__ gin, const E* __restrict__ w, const E* __restrict__ Tm,
    const float* S0, E* __restrict__ o, float* S_T, E* __restrict__ Sc, int BH, int T, int DV,
    int NC, Packed pk, SegPlan seg) {
    __shared__ __align__(16) StateLds<E, DK, DVT, C> L;
    const int ntile = SEG ? seg.ntv + seg.nta : DV / DVT;
    const int L_ = blockIdx.x, per = 8 * ntile;
    const int unit = (L_ / per) * 8 + (L_ % 8), tile = (L_ % per) / 8;
    if constexpr (SEG && !OUT) {
        if (L_ >= seg.map_wgs) {
            // segment 0 starts from S0: its value tiles run it with read-out
            // (and keep its end state); it has no map to form
            const int i = L_ - seg.map_wgs, per0 = 8 * seg.ntv;
            const int head = (i / per0) * 8 + (i % 8);
            if (head >= BH) return;
            state_body<E, DK, DVT, C, VL, true, true>(L, q, k, v, gin, w, Tm, S0, o, S_T, Sc, T,
                                                      DV, NC, pk, seg, head, 0, (i % per0) / 8);
            return;
        }
        const int units = BH * (seg.nseg - 2);  // the maps of segments 1 .. nseg - 2
        for (int r = 0; r < seg.map_jobs; ++r) {
            const int i = L_ + r * seg.map_wgs;
            const int u = (i / per) * 8 + (i % 8);
            if (u >= units) continue;
            if (r > 0) sync_lds();  // the previous job's last LDS reads are done
            state_body<E, DK, DVT, C, VL, false, true>(L, q, k, v, gin, w, Tm, S0, o, S_T, Sc, T,
                                                       DV, NC, pk, seg, u % BH, 1 + u / BH,
                                                       (i % per) / 8);
        }
    } else if constexpr (SEG) {
        if (unit >= BH * seg.nsegL) return;
        state_body<E, DK, DVT, C, VL, true, true>(L, q, k, v, gin, w, Tm, S0, o, S_T, Sc, T, DV,
                                                  NC, pk, seg, unit % BH, seg.g0 + unit / BH, tile);
    } else {
        if (unit >= BH) return;
        state_body<E, DK, DVT, C, VL, OUT, false>(L, q, k, v, gin, w, Tm, S0, o, S_T, Sc, T, DV,
                                                  NC, pk, seg, unit, 0, tile);
    }
}

// Start states of the segments: S_{g+1} = S_g A_g + B_g for g = 1 .. nseg - 2,
// in order.  On entry Sseg[1] holds the true end state of segment 0 and
// Sseg[g + 1] (g >= 1) the end state B_g of segment g from a zero start;
// Aseg[g] holds A_g (d_k x d_k).  One workgroup of 8 waves per (kCombRows rows
// of S, head), fp32 throughout.  A_g sits in LDS; A_{g+1} and the rows of
// B_{g+1} are loaded (every load issued at once) while step g computes, so the
// steps do not wait for global memory.
constexpr int kCombThreads = 512;
template <int DK> constexpr int comb_rows() { return DK >= 64 ? 8 : kCombThreads / DK; }

template <int DK>
__global__ __launch_bounds__(kCombThreads) void seg_combine_kernel(float* __restrict__ Sseg,
                                                                  const float* __restrict__ Aseg,
                                                                  int DV, int nseg) {
    constexpr int R = comb_rows<DK>(), RG = kCombThreads / DK, RPT = R / RG;  // rows per thread
    constexpr int NA = DK * DK / 4;                             // float4 pieces of A
    constexpr int NV = (NA + kCombThreads - 1) / kCombThreads;  // ... per thread
    static_assert(RPT * RG == R && RPT >= 1, "combine tiling");
    __shared__ __align__(16) float sA[2][DK * DK];
    __shared__ __align__(16) float sS[R][DK];
    const int tid = threadIdx.x, i = tid % DK, rg = tid / DK;
    const size_t bh = blockIdx.y;
    const int j0 = blockIdx.x * R;
    float* base = Sseg + bh * (size_t)nseg * DV * DK;
    const float* abase = Aseg + bh * (size_t)nseg * DK * DK;
    // A_{g+1} is prefetched into eight named registers: held in an array,
    // even one indexed with constants only, the compiler kept it in scratch
    // memory (a stack round trip per step)
    static_assert(NV <= 8, "combine prefetch registers");
    [[maybe_unused]] float4 pa0, pa1, pa2, pa3, pa4, pa5, pa6, pa7;
    float preB[RPT];
#define KDN_COMB_LD(X)                                                                   \
    if constexpr (X < NV)                                                                \
        if (NA % kCombThreads == 0 || tid + kCombThreads * X < NA)                       \
            pa##X = src[tid + kCombThreads * X];
#define KDN_COMB_ST(X)                                                                   \
    if constexpr (X < NV)                                                                \
        if (NA % kCombThreads == 0 || tid + kCombThreads * X < NA)                       \
            dst[tid + kCombThreads * X] = pa##X;
#define KDN_COMB_FETCH(G_)                                                                   \
    {                                                                                        \
        const float4* src = reinterpret_cast<const float4*>(abase + (size_t)(G_) * DK * DK); \
        KDN_COMB_LD(0) KDN_COMB_LD(1) KDN_COMB_LD(2) KDN_COMB_LD(3)                          \
        KDN_COMB_LD(4) KDN_COMB_LD(5) KDN_COMB_LD(6) KDN_COMB_LD(7)                          \
        const float* bsrc = base + ((size_t)((G_) + 1) * DV + j0) * DK;                      \
        _Pragma("unroll") for (int r = 0; r < RPT; ++r) preB[r] =                            \
            bsrc[(size_t)(rg * RPT + r) * DK + i];                                           \
    }
#define KDN_COMB_STAGE(BUF_)                                                                 \
    {                                                                                        \
        float4* dst = reinterpret_cast<float4*>(sA[BUF_]);                                   \
        KDN_COMB_ST(0) KDN_COMB_ST(1) KDN_COMB_ST(2) KDN_COMB_ST(3)                          \
        KDN_COMB_ST(4) KDN_COMB_ST(5) KDN_COMB_ST(6) KDN_COMB_ST(7)                          \
    }
    KDN_COMB_FETCH(1)
    for (int e = tid; e < R * DK; e += kCombThreads)
        sS[e / DK][e % DK] = base[((size_t)1 * DV + j0 + e / DK) * DK + e % DK];
    KDN_COMB_STAGE(1)
    __syncthreads();
    for (int g = 1; g + 1 < nseg; ++g) {
        float acc[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) acc[r] = preB[r];
        if (g + 2 < nseg) KDN_COMB_FETCH(g + 1)  // in flight during this step
        float* out = base + ((size_t)(g + 1) * DV + j0) * DK;
        const float* A = sA[g & 1];
#pragma unroll 4
        for (int m = 0; m < DK; m += 4) {
            const float a0 = A[(m + 0) * DK + i], a1 = A[(m + 1) * DK + i];
            const float a2 = A[(m + 2) * DK + i], a3 = A[(m + 3) * DK + i];
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const float4 sv = *reinterpret_cast<const float4*>(&sS[rg * RPT + r][m]);
                acc[r] = fmaf(sv.x, a0, acc[r]);
                acc[r] = fmaf(sv.y, a1, acc[r]);
                acc[r] = fmaf(sv.z, a2, acc[r]);
                acc[r] = fmaf(sv.w, a3, acc[r]);
            }
        }
        __syncthreads();  // every thread is done reading S_g and A_g
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            out[(size_t)(rg * RPT + r) * DK + i] = acc[r];
            sS[rg * RPT + r][i] = acc[r];
        }
        if (g + 2 < nseg) KDN_COMB_STAGE((g + 1) & 1)
        __syncthreads();
    }
#undef KDN_COMB_FETCH
#undef KDN_COMB_STAGE
#undef KDN_COMB_LD
#undef KDN_COMB_ST
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

template <typename E, typename G, int DK, int C>
hipError_t prep_t(const Shape& s, bool fuse, const void* k, const void* a, const void* nu,
                  const void* r, const float* lc, const float* agg, void* w, void* Tm, float* g,
                  float* dinv, hipStream_t st) {
    static_assert(PrepLds<E, DK, C>::BYTES <= kLdsLimit, "prep LDS");
    const dim3 grid((s.nc + 1) / 2, s.BH);
#define KDN_PREP_L(FUSE_, VL_)                                                                \
    launch_k((prep_kernel<E, G, DK, C, FUSE_, VL_>), grid, dim3(kThreads), 0, st,            \
             static_cast<const E*>(k), static_cast<const G*>(a), static_cast<const G*>(nu),  \
             static_cast<const G*>(r), s.diag, lc, reinterpret_cast<const float4*>(agg),         \
             static_cast<E*>(w), static_cast<E*>(Tm), g,                                         \
             dinv, s.T, s.nc, s.pk)
    if (s.varlen) {
        if (!fuse) return hipErrorInvalidValue;  // packed batches: the forward only
        KDN_PREP_L(true, true);
    } else if (fuse) {
        KDN_PREP_L(true, false);
    } else {
        KDN_PREP_L(false, false);
    }
#undef KDN_PREP_L
    return hipGetLastError();
}

template <typename E, int DK, int DVT, int C>
hipError_t state_t(const Shape& s, const void* q, const void* k, const void* v, const float* g,
                   const void* w, const void* Tm, const float* S0, void* o, float* S_T, void* Sc,
                   const SegWs* sw, hipStream_t st) {
    if constexpr (state_fits<E, DK, DVT, C>()) {
        const dim3 block(StateCfg<E, DK, DVT, C>::THREADS);
        const int ntv = s.dv / DVT;
        auto grid = [](int units, int ntile) { return dim3((units + 7) / 8 * 8 * ntile); };
#define KDN_STATE_L(VL_, OUT_, SEG_, GRID_, PLAN_)                                            \
    launch_k((state_kernel<E, DK, DVT, C, VL_, OUT_, SEG_>), GRID_, block, 0, st,             \
             static_cast<const E*>(q), static_cast<const E*>(k), static_cast<const E*>(v), g,  \
             static_cast<const E*>(w), static_cast<const E*>(Tm), S0, static_cast<E*>(o), S_T, \
             static_cast<E*>(Sc), s.BH, s.T, s.dv, s.nc, s.pk, PLAN_)
        const SegPlan plain;
        if (!sw || sw->nseg <= 1 || Sc || !o) {
            if (s.varlen) KDN_STATE_L(true, true, false, grid(s.BH, ntv), plain);
            else if (o) KDN_STATE_L(false, true, false, grid(s.BH, ntv), plain);
            else KDN_STATE_L(false, false, false, grid(s.BH, ntv), plain);
        } else {
            // segments: segment 0 with read-out beside the maps of segments
            // 1 .. nseg - 2, their composition into every segment's start
            // state, then the read-out of segments 1 .. nseg - 1; the caller's
            // timing events bracket the three launches
            const LaunchTiming t = launch_timing();
            SegPlan p;
            p.nseg = sw->nseg;
            p.Lc = sw->Lc;
            p.L0 = sw->L0 > 0 ? sw->L0 : sw->Lc;
            p.Sseg = sw->Sseg;
            p.Aseg = sw->Aseg;
            p.g0 = 0;
            p.nsegL = sw->nseg - 1;
            p.ntv = ntv;
            p.nta = (DK + DVT - 1) / DVT;  // identity rows past d_k are not written
            // the maps launch: segment 0's value tiles, and as many map
            // workgroups as the other CUs hold, each taking the fewest jobs
            // that cover the maps (a whole number of units per round if that fits)
            const int per = 8 * (p.ntv + p.nta);
            const long jobs = (long)(s.BH * (sw->nseg - 2) + 7) / 8 * per;
            const int nv0 = (s.BH + 7) / 8 * 8 * ntv;
            const int avail = std::max(8, (kStateCUs - nv0) / 8 * 8);
            p.map_jobs = jobs > 0 ? static_cast<int>((jobs + avail - 1) / avail) : 0;
            p.map_wgs = jobs > 0 ? static_cast<int>((jobs + p.map_jobs - 1) / p.map_jobs) : 0;
            p.map_wgs = (p.map_wgs + per - 1) / per * per <= avail
                            ? (p.map_wgs + per - 1) / per * per
                            : (p.map_wgs + 7) / 8 * 8;
            const dim3 gmaps(p.map_wgs + nv0);
            launch_timing() = LaunchTiming{t.start, nullptr};
            if (s.varlen) KDN_STATE_L(true, false, true, gmaps, p);
            else KDN_STATE_L(false, false, true, gmaps, p);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            if (sw->nseg > 2) {
                launch_k(seg_combine_kernel<DK>, dim3(s.dv / comb_rows<DK>(), s.BH), dim3(kCombThreads), 0, st,
                         sw->Sseg, static_cast<const float*>(sw->Aseg), s.dv, sw->nseg);
                e = hipGetLastError();
                if (e != hipSuccess) return e;
            }
            p.g0 = 1;
            p.nsegL = sw->nseg - 1;
            p.nta = 0;
            launch_timing() = LaunchTiming{nullptr, t.stop};
            if (s.varlen) KDN_STATE_L(true, true, true, grid(s.BH * p.nsegL, p.ntv), p);
            else KDN_STATE_L(false, true, true, grid(s.BH * p.nsegL, p.ntv), p);
        }
#undef KDN_STATE_L
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <typename E>
hipError_t prep_e(const Shape& s, bool fuse, const void* k, const void* a, const void* nu,
                  const void* r, const float* lc, const float* agg, void* w, void* Tm, float* g,
                  float* dinv, hipStream_t st) {
#define KDN_PREP(DK_, C_)                                                                   \
    if (s.dk == DK_ && s.chunk == C_)                                                       \
        return s.gate_bf16                                                                  \
                   ? prep_t<E, bf16_t, DK_, C_>(s, fuse, k, a, nu, r, lc, agg, w, Tm, g, dinv, st) \
                   : prep_t<E, float, DK_, C_>(s, fuse, k, a, nu, r, lc, agg, w, Tm, g, dinv, st);
#define KDN_PREP_C(DK_) KDN_PREP(DK_, 16) KDN_PREP(DK_, 32) KDN_PREP(DK_, 64)
    KDN_PREP_C(32) KDN_PREP_C(64) KDN_PREP_C(128)
#undef KDN_PREP_C
#undef KDN_PREP
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t state_e(const Shape& s, const void* q, const void* k, const void* v, const float* g,
                   const void* w, const void* Tm, const float* S0, void* o, float* S_T, void* Sc,
                   const SegWs* sw, hipStream_t st) {
    const int dvt = dv_tile(s);
#define KDN_ST(DK_, DVT_, C_)                                                             \
    if (s.dk == DK_ && dvt == DVT_ && s.chunk == C_)                                      \
        return state_t<E, DK_, DVT_, C_>(s, q, k, v, g, w, Tm, S0, o, S_T, Sc, sw, st);
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
                             const void* nu, const void* r, const float* lam_chunk,
                             const float* agg, void* w, void* Tm, float* g, hipStream_t st,
                             float* dinv) {
    if (s.BH == 0 || s.nc == 0) return hipSuccess;
    if (fuse_gain && s.diag && !agg) return hipErrorInvalidValue;
    return s.qkv_bf16
               ? prep_e<bf16_t>(s, fuse_gain, k, a, nu, r, lam_chunk, agg, w, Tm, g, dinv, st)
               : prep_e<float>(s, fuse_gain, k, a, nu, r, lam_chunk, agg, w, Tm, g, dinv, st);
}

hipError_t launch_chunk_state(const Shape& s, const void* q, const void* k, const void* v,
                              const float* g, const void* w, const void* Tm, const float* S0,
                              void* o, float* S_T, hipStream_t st, void* Sc, const SegWs* seg) {
    if (s.BH == 0) return hipSuccess;
    return s.qkv_bf16 ? state_e<bf16_t>(s, q, k, v, g, w, Tm, S0, o, S_T, Sc, seg, st)
                      : state_e<float>(s, q, k, v, g, w, Tm, S0, o, S_T, Sc, seg, st);
}

// The segmented pass costs, in time: the maps launch (segment 0 with read-out
// on BH * ntv CUs, beside rounds of the other segments' maps on the remaining
// CUs), the composition (nseg - 2 dependent steps) and the read-out launch
// (rounds of segments 1 .. nseg - 1).  Per chunk a map step takes about 1.6 us
// and a read-out step 2.5 us (d 128, chunk 64, one workgroup per CU), a
// composition step about 3.5 us, and the two extra launches about 5 us.  Given
// nseg, segment 0 is made as long as the maps rounds beside it take, the other
// segments share the rest; the plan with the least estimated time wins, the
// plain pass (2.5 us per chunk on one round) included.
SegSplit state_split(const Shape& s) {
    SegSplit best{1, s.nc, s.nc};
    const int dvt = dv_tile(s);
    if (s.BH <= 0 || dvt <= 0 || s.nc < 16) return best;
    constexpr double kMap = 1.6, kRead = 2.5, kComb = 3.5, kLaunch = 5.0;
    constexpr int kCUs = kStateCUs, kMinLen = 2;
    const int ntv = s.dv / dvt, nta = (s.dk + dvt - 1) / dvt;
    const long seg0 = (long)s.BH * ntv;  // segment 0's workgroups in the maps launch
    if (seg0 >= kCUs / 2) return best;   // enough heads to fill the GPU
    double best_t = kRead * s.nc;
    for (int n = 3; n <= 64 && (n - 1) * kMinLen + kMinLen <= s.nc; ++n) {
        const long maps = (long)s.BH * (n - 2) * (ntv + nta);
        const long rm = (maps + (kCUs - seg0) - 1) / (kCUs - seg0);
        const long rr = ((long)s.BH * (n - 1) * ntv + kCUs - 1) / kCUs;
        const double rho = kMap * rm / kRead;  // segment 0's length over the others'
        const int Lc = static_cast<int>(std::ceil(s.nc / (rho + n - 1)));
        const int L0 = s.nc - (n - 1) * Lc;
        if (L0 < kMinLen || Lc < kMinLen) continue;
        const double t = std::max(kRead * L0, kMap * rm * Lc) + kRead * rr * Lc +
                         kComb * (n - 2) + kLaunch;
        if (t < best_t) {
            best_t = t;
            best = SegSplit{n, Lc, L0};
        }
    }
    return best;
}

}  // namespace kdn
