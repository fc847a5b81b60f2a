// kdn_tiles.h -- register/LDS tile helpers shared by the chunkwise forward
// kernels and the backward kernels (gfx950 only): vector packing of MFMA
// result tiles, the per-chunk operand loads of the sequential state passes and
// their staging into LDS.
#pragma once

#include "kdn_device.h"
#include "kdn_launch.h"

namespace kdn {
namespace {

constexpr int cmax(int x, int y) { return x > y ? x : y; }
constexpr int cmin(int x, int y) { return x < y ? x : y; }

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
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
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

// Two 16x16 MFMA result tiles that neighbour along their 4-consecutive
// dimension (lane l holds elements 4 (l / 16) .. +3 of line l % 16 in each),
// written as 16-byte stores: the lanes of each pair of 16-lane rows swap halves
// (v_permlane16_swap), after which lanes of even rows hold 8 consecutive
// elements of tile 0 and lanes of odd rows 8 of tile 1.  p0 / p1: the start of
// the lane's line in tile 0 / tile 1.
template <typename E>
__device__ __forceinline__ void store8x2(E* p0, E* p1, floatx4 a, floatx4 b, int lane);
template <>
__device__ __forceinline__ void store8x2<float>(float* p0, float* p1, floatx4 a, floatx4 b,
                                                int lane) {
    store4<float>(p0 + 4 * (lane >> 4), a[0], a[1], a[2], a[3]);
    store4<float>(p1 + 4 * (lane >> 4), b[0], b[1], b[2], b[3]);
}
template <>
__device__ __forceinline__ void store8x2<bf16_t>(bf16_t* p0, bf16_t* p1, floatx4 a, floatx4 b,
                                                 int lane) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 s0 = __builtin_amdgcn_permlane16_swap(pack_bf16(a[0], a[1]),
                                                      pack_bf16(b[0], b[1]), false, false);
    const u32x2 s1 = __builtin_amdgcn_permlane16_swap(pack_bf16(a[2], a[3]),
                                                      pack_bf16(b[2], b[3]), false, false);
    const int g = lane >> 4;
    bf16_t* dst = ((g & 1) ? p1 : p0) + 8 * (g >> 1);
    *reinterpret_cast<u32x4*>(dst) = u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// the same, with the store predicated per lane (the swap involves every lane;
// a lane stores the line it held before the swap, so its predicate is its own)
template <typename E>
__device__ __forceinline__ void store8x2_if(bool pred, E* p0, E* p1, floatx4 a, floatx4 b,
                                            int lane);
template <>
__device__ __forceinline__ void store8x2_if<float>(bool pred, float* p0, float* p1, floatx4 a,
                                                   floatx4 b, int lane) {
    if (pred) store8x2<float>(p0, p1, a, b, lane);
}
template <>
__device__ __forceinline__ void store8x2_if<bf16_t>(bool pred, bf16_t* p0, bf16_t* p1, floatx4 a,
                                                    floatx4 b, int lane) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 s0 = __builtin_amdgcn_permlane16_swap(pack_bf16(a[0], a[1]),
                                                      pack_bf16(b[0], b[1]), false, false);
    const u32x2 s1 = __builtin_amdgcn_permlane16_swap(pack_bf16(a[2], a[3]),
                                                      pack_bf16(b[2], b[3]), false, false);
    const int g = lane >> 4;
    bf16_t* dst = ((g & 1) ? p1 : p0) + 8 * (g >> 1);
    if (pred) *reinterpret_cast<u32x4*>(dst) = u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// The inverse of store8x2: two neighbouring tiles read with 16-byte loads and
// returned in the MFMA result layout (lane l: elements 4 (l / 16) .. +3 of its
// line in each tile); the swap is its own inverse.
template <typename E>
__device__ __forceinline__ void load8x2(const E* p0, const E* p1, float (&a)[4], float (&b)[4],
                                        int lane);
template <>
__device__ __forceinline__ void load8x2<float>(const float* p0, const float* p1, float (&a)[4],
                                               float (&b)[4], int lane) {
    load4<float>(p0 + 4 * (lane >> 4), a);
    load4<float>(p1 + 4 * (lane >> 4), b);
}
template <>
__device__ __forceinline__ void load8x2<bf16_t>(const bf16_t* p0, const bf16_t* p1,
                                                float (&a)[4], float (&b)[4], int lane) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const int g = lane >> 4;
    const u32x4 v = *reinterpret_cast<const u32x4*>(((g & 1) ? p1 : p0) + 8 * (g >> 1));
    const u32x2 s0 = __builtin_amdgcn_permlane16_swap(v[0], v[2], false, false);
    const u32x2 s1 = __builtin_amdgcn_permlane16_swap(v[1], v[3], false, false);
    a[0] = __uint_as_float(s0[0] << 16);
    a[1] = __uint_as_float(s0[0] & 0xFFFF0000u);
    a[2] = __uint_as_float(s1[0] << 16);
    a[3] = __uint_as_float(s1[0] & 0xFFFF0000u);
    b[0] = __uint_as_float(s0[1] << 16);
    b[1] = __uint_as_float(s0[1] & 0xFFFF0000u);
    b[2] = __uint_as_float(s1[1] << 16);
    b[3] = __uint_as_float(s1[1] & 0xFFFF0000u);
}

// inclusive prefix sum over the 64 lanes of a wave, in DPP moves: row_shr 1,
// 2, 4, 8 (lanes shifted in from outside the row of 16 read 0) give every row's
// own prefix; row_bcast 15 adds the last lane of row 0 to row 1 and of row 2 to
// row 3, then row_bcast 31 adds lane 31 (the sum of rows 0-1) to rows 2 and 3.
// Rows a move leaves out (its row mask) receive the `old` operand, 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float wave_incl_sum(float x) {
    x += dpp_or_zero<0x111, 0xF>(x);
    x += dpp_or_zero<0x112, 0xF>(x);
    x += dpp_or_zero<0x114, 0xF>(x);
    x += dpp_or_zero<0x118, 0xF>(x);
    x += dpp_or_zero<0x142, 0xA>(x);
    x += dpp_or_zero<0x143, 0xC>(x);
    return x;
}

template <typename E, int DK, int DVT, int C> struct StateCfg {
    static constexpr int NW = 8, THREADS = 64 * NW;
    // rows padded by 32 bytes: a row stride of 8 (mod 16) dwords lets the MFMA
    // fragment reads (16 rows x 4 column groups) run at full LDS bandwidth
    static constexpr int PAD = 32 / (int)sizeof(E), VEC = Vec16<E>::N;
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
        (4 * C * LDK + DVT * LDK + C * LDV + 2 * DVT * LDC + 2 * C * LDC + C * LDV) *
            (int)sizeof(E) +
        6 * C * (int)sizeof(float);  // two sets of the three decay tables
};

// Loads of one chunk into registers, two chunks before its use, and their
// staging into LDS.  The loads never branch on their results, so that the waits
// for them can be counted exactly and placed at the staging: a chunk past the
// end reloads the last one and rows past the end of the sequence load the last
// valid row (those rows only reach outputs that are never stored, except
// through W, whose padded rows are stored as zeros).  The loads come in three
// parts issued at the starts of the three phases of a chunk: a burst of every
// wave's loads at once would stall the waves on the vector-memory issue queue.
// WQ = false: Q is neither loaded nor staged (a pass with no read-out).
enum { kLoadKQ = 0, kLoadW = 1, kLoadVTG = 2, kLoadAll = 3 };
template <typename E, int DK, int DVT, int C, int PART, bool WQ = true>
__device__ __forceinline__ void state_prefetch(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ w, const E* __restrict__ Tm, const float* __restrict__ gin,
    const Slab& sl, int j0, int DV, int cc, int tid, int lane,
    u32x4 (&pk)[StateCfg<E, DK, DVT, C>::PK], u32x4 (&pq)[StateCfg<E, DK, DVT, C>::PK],
    u32x4 (&pw)[StateCfg<E, DK, DVT, C>::PK], u32x4 (&pv)[StateCfg<E, DK, DVT, C>::PV],
    u32x4 (&pt)[StateCfg<E, DK, DVT, C>::PT], float& pg) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int VEC = G::VEC;
    const int c = min(cc, sl.nc - 1);
    const int t0 = c * C, n = min(C, sl.T - t0);
    const size_t row0 = sl.row0 + t0;
    if constexpr (PART == kLoadKQ || PART == kLoadW || PART == kLoadAll) {
#pragma unroll
        for (int x = 0; x < G::PK; ++x) {
            const int e = tid + G::THREADS * x;
            if (G::NVK % G::THREADS == 0 || e < G::NVK) {
                const int t = e / (DK / VEC), c0 = (e % (DK / VEC)) * VEC;
                const size_t off = (row0 + min(t, n - 1)) * DK + c0;
                if constexpr (PART != kLoadW) {
                    pk[x] = *reinterpret_cast<const u32x4*>(k + off);
                    if constexpr (WQ) pq[x] = *reinterpret_cast<const u32x4*>(q + off);
                }
                if constexpr (PART != kLoadKQ) pw[x] = *reinterpret_cast<const u32x4*>(w + off);
            }
        }
    }
    if constexpr (PART == kLoadVTG || PART == kLoadAll) {
#pragma unroll
        for (int x = 0; x < G::PV; ++x) {
            const int e = tid + G::THREADS * x;
            if (G::NVV % G::THREADS == 0 || e < G::NVV) {
                const int t = e / (DVT / VEC), c0 = (e % (DVT / VEC)) * VEC;
                pv[x] = *reinterpret_cast<const u32x4*>(v + (row0 + min(t, n - 1)) * DV + j0 + c0);
            }
        }
        const E* Tc = Tm + (sl.c0 + c) * (size_t)(C * C);
#pragma unroll
        for (int x = 0; x < G::PT; ++x) {
            const int e = tid + G::THREADS * x;
            if (G::NVT % G::THREADS == 0 || e < G::NVT)
                pt[x] = *reinterpret_cast<const u32x4*>(Tc + e * VEC);
        }
        // chunk-local cumulative log2 decay (padding rows repeat the last value)
        pg = gin[(sl.c0 + c) * C + min(lane, C - 1)];
    }
}

// parts of a chunk staged from registers into LDS: K, Q, W and V; T and the
// decay tables.  zero_v: V is staged as zeros (the loaded values are dropped).
// parts: K, Q, W, V; the T matrix; the decay tables (g, gamma, gamma_C / gamma)
enum { kStageKQWV = 1, kStageTm = 2, kStageTab = 4, kStageT = 6, kStageAll = 7 };
template <typename E, int DK, int DVT, int C, int PARTS, bool WQ = true>
__device__ __forceinline__ void state_stage(
    E* sK, E* sQ, E* sWc, E* sV, E* sT, float* sg, float* sgam, float* sdel, int n, int tid,
    int lane, int wave, const u32x4 (&pk)[StateCfg<E, DK, DVT, C>::PK],
    const u32x4 (&pq)[StateCfg<E, DK, DVT, C>::PK], const u32x4 (&pw)[StateCfg<E, DK, DVT, C>::PK],
    const u32x4 (&pv)[StateCfg<E, DK, DVT, C>::PV], const u32x4 (&pt)[StateCfg<E, DK, DVT, C>::PT],
    float pg, bool zero_v = false) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int VEC = G::VEC, LDK = G::LDK, LDC = G::LDC, LDV = G::LDV;
    if constexpr ((PARTS & kStageKQWV) != 0) {
#pragma unroll
        for (int x = 0; x < G::PK; ++x) {
            const int e = tid + G::THREADS * x;
            if (G::NVK % G::THREADS == 0 || e < G::NVK) {
                const int t = e / (DK / VEC), c0 = (e % (DK / VEC)) * VEC;
                *reinterpret_cast<u32x4*>(sK + t * LDK + c0) = pk[x];
                if constexpr (WQ) *reinterpret_cast<u32x4*>(sQ + t * LDK + c0) = pq[x];
                // padded rows of W are zero (a select at staging time, when the
                // loaded row has to have arrived anyway)
                const u32x4 zero = {0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(sWc + t * LDK + c0) = (t < n) ? pw[x] : zero;
            }
        }
#pragma unroll
        for (int x = 0; x < G::PV; ++x) {
            const int e = tid + G::THREADS * x;
            if (G::NVV % G::THREADS == 0 || e < G::NVV) {
                const int t = e / (DVT / VEC), c0 = (e % (DVT / VEC)) * VEC;
                const u32x4 zero = {0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(sV + t * LDV + c0) = zero_v ? zero : pv[x];
            }
        }
    }
    if constexpr ((PARTS & kStageTm) != 0) {
#pragma unroll
        for (int x = 0; x < G::PT; ++x) {
            const int e = tid + G::THREADS * x;
            if (G::NVT % G::THREADS == 0 || e < G::NVT) {
                const int t = e / (C / VEC), c0 = (e % (C / VEC)) * VEC;
                *reinterpret_cast<u32x4*>(sT + t * LDC + c0) = pt[x];
            }
        }
    }
    if constexpr ((PARTS & kStageTab) != 0) {
        if (wave == 0) {
            const float glast = lane_value(pg, C - 1);
            if (lane < C) {
                sg[lane] = pg;
                sgam[lane] = exp2_hw(pg);
                sdel[lane] = exp2_hw(glast - pg);
            }
        }
    }
}

// the wave's share of the state, S^T blocks (BI x BV tiles); element e <->
// i = 16 ti + 4 (lane/16) + e, j = 16 tj + lane % 16
template <typename E, int DK, int DVT, int C>
using StateAcc = floatx4[StateCfg<E, DK, DVT, C>::SPW][StateCfg<E, DK, DVT, C>::BI]
                        [StateCfg<E, DK, DVT, C>::BV];

// S^T blocks of the state -> LDS operand S[j][i] in qkv dtype
template <typename E, int DK, int DVT, int C>
__device__ __forceinline__ void state_write(const StateAcc<E, DK, DVT, C>& accS, E* sS, int wave,
                                            int lane) {
    using G = StateCfg<E, DK, DVT, C>;
#pragma unroll
    for (int x = 0; x < G::SPW; ++x) {
        const int job = wave + G::NW * x;
        if (job < G::NSJ) {
            const int ib = (job / G::NVB) * G::BI, jb = (job % G::NVB) * G::BV;
            static_assert(G::BI == 2, "state tiles pair along i");
#pragma unroll
            for (int bv = 0; bv < G::BV; ++bv) {
                E* row = sS + (16 * (jb + bv) + (lane & 15)) * G::LDK + 16 * ib;
                store8x2<E>(row, row + 16, accS[x][0][bv], accS[x][1][bv], lane);
            }
        }
    }
}

// v[j] summed over the 16 lanes of each 16-lane group: on return lane l holds
// in v[0] the group total of v[l % 16] (15 exchanges instead of 16 reductions).
// Step H pairs every lane with one whose bit H differs and whose higher bits
// agree: the lane keeps the half of its values selected by its own bit H and
// adds the partner's copy of that half.  Lane l therefore ends with index
// l % 16 whatever the pairing, so each step uses the DPP move that pairs such
// lanes within the row of 16: row_mirror (l <-> 15 - l) for bit 3,
// row_half_mirror (l <-> 7 - l in each 8) for bit 2, quad permutes (xor 2,
// xor 1) for bits 1 and 0 -- one VALU move each, no LDS traffic.
template <int H, int CTRL>
__device__ __forceinline__ void transpose_sum_step(float (&v)[16], int lane) {
    const bool upper = (lane & H) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const float keep = upper ? v[j + H] : v[j];
        const float send = upper ? v[j] : v[j + H];
        v[j] = keep + dpp<CTRL>(send);
    }
}
__device__ __forceinline__ float transpose_sum16(float (&v)[16], int lane) {
    transpose_sum_step<8, 0x140>(v, lane);  // row_mirror
    transpose_sum_step<4, 0x141>(v, lane);  // row_half_mirror
    transpose_sum_step<2, 0x4E>(v, lane);   // quad_perm [2, 3, 0, 1]
    transpose_sum_step<1, 0xB1>(v, lane);   // quad_perm [1, 0, 3, 2]
    return v[0];
}

// The LDS operand copy of the state, S[j][i] (DVT rows of stride LDK), to
// global rows of stride DK with 16-byte stores (whole rows per 16-lane group)
template <typename E, int DK, int DVT, int C>
__device__ __forceinline__ void state_copy_out(const E* sS, E* dst, int tid) {
    using G = StateCfg<E, DK, DVT, C>;
    constexpr int VPR = DK / G::VEC, NV = DVT * VPR;
#pragma unroll
    for (int x = 0; x < (NV + G::THREADS - 1) / G::THREADS; ++x) {
        const int e = tid + G::THREADS * x;
        if (NV % G::THREADS == 0 || e < NV) {
            const int j = e / VPR, c0 = (e % VPR) * G::VEC;
            *reinterpret_cast<u32x4*>(dst + j * DK + c0) =
                *reinterpret_cast<const u32x4*>(sS + j * G::LDK + c0);
        }
    }
}

}  // namespace
}  // namespace kdn
