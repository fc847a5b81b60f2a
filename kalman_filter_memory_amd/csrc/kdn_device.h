// kdn_device.h -- device helpers shared by the libkdn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdn {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef float floatx4 __attribute__((ext_vector_type(4)));
// 16-byte register payload of a vector load; a native vector type (not the HIP
// uint4 struct, whose copies become memcpys that can pin arrays of them to
// scratch memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short short4x __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ bf16_t f2bf(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}
// two floats -> two bfloat16 packed in one word (x in the low half)
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float float2_t __attribute__((ext_vector_type(2)));
    const float2_t v = {x, y};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename E> __device__ __forceinline__ float to_f(E x);
template <> __device__ __forceinline__ float to_f<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t x) { return bf2f(x); }

template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float x) { return f2bf(x); }

// Load one element of a gate tensor whose dtype is only known at run time.
__device__ __forceinline__ float load_gate(const void* p, size_t i, bool bf16) {
    return bf16 ? bf2f(static_cast<const bf16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// ------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations
// and meets the other waves, without waiting for outstanding global loads (a
// full __syncthreads() also drains vmcnt, which would expose the latency of
// loads issued early for the next chunk).
__device__ __forceinline__ void sync_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// fast reciprocal (v_rcp_f32, about 1 ulp)
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32, about 1 ulp)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
// value of lane `l` (uniform) of x, broadcast through a scalar register
// index of the calling wave in its workgroup, in a scalar register: the
// compiler's divergence analysis cannot see that threadIdx.x / 64 is uniform
// across a wave, and would otherwise keep everything derived from it (tile
// choices, row offsets, addresses) in vector registers
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Raw buffer resource over `bytes` bytes at p (descriptor word 3 of the gfx9
// family: 32-bit data format, no swizzle).  Buffer loads take a per-lane
// offset in a vector register and a uniform one in a scalar register, so rows
// chosen uniformly cost no vector address arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ float lane_value(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// N contiguous elements of E at p as floats, in vector loads (p aligned to
// N * sizeof(E) bytes, or to 16 when that is more; N * sizeof(E) a power of two
// of at least 4 bytes)
template <typename E, int N>
__device__ __forceinline__ void load_vec(const E* p, float* f) {
    constexpr int W = N * int(sizeof(E)) / 4;  // 32-bit words
    uint32_t u[W];
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int i = 0; i < W / 4; ++i) {
            const u32x4 x = reinterpret_cast<const u32x4*>(p)[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) u[4 * i + j] = x[j];
        }
    } else if constexpr (W == 2) {
        typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
        const u32x2_t x = *reinterpret_cast<const u32x2_t*>(p);
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

// x of another lane of the same row of 16, chosen by a DPP control (quad_perm,
// row_mirror, row_half_mirror ...), as a source modifier of one VALU move
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the LPR aligned lanes of a row group, returned to every lane of it,
// without LDS: quad_perm xor 1 and xor 2, then row_half_mirror (other quad of 8
// lanes), row_mirror (other 8 of 16) and, for 32 lanes, v_permlane16_swap of x
// with itself, whose two results add up to x + x of the lane 16 away.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
template <int LPR> __device__ __forceinline__ float group_sum(float x) {
    static_assert(LPR == 2 || LPR == 4 || LPR == 8 || LPR == 16 || LPR == 32,
                  "unsupported group");
    x += dpp<0xB1>(x);
    if constexpr (LPR >= 4) x += dpp<0x4E>(x);
    if constexpr (LPR >= 8) x += dpp<0x141>(x);
    if constexpr (LPR >= 16) x += dpp<0x140>(x);
    if constexpr (LPR >= 32) {
        const u32x2 s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                         false, false);
        x = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    }
    return x;
}

// ------------------------------------------------------------------- MFMA
// 16x16 output tiles.  Operand fragments are read from row-major LDS arrays
// whose contraction index is contiguous:  A as [m][k], B as [n][k].
// Output (C) layout of one 16x16 tile for lane l:  element e (0..3) holds
// C[4*(l/16) + e][l % 16].
template <typename E> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KS = 32;  // contraction depth of one instruction
    typedef bf16x8 frag_t;
    typedef short4x frag16_t;
    // lane l reads 8 consecutive k at row (l % 16), k offset 8 * (l / 16)
    static __device__ __forceinline__ bf16x8 frag(const bf16_t* base, int ld, int row0, int k0,
                                                  int lane) {
        const bf16_t* p = base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
        return *reinterpret_cast<const bf16x8*>(p);
    }
    static __device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // 16-deep step (v_mfma_f32_16x16x16_bf16): lane l reads 4 consecutive k at
    // row (l % 16), k offset 4 * (l / 16)
    static __device__ __forceinline__ short4x frag16(const bf16_t* base, int ld, int row0,
                                                     int k0, int lane) {
        return *reinterpret_cast<const short4x*>(base + (row0 + (lane & 15)) * ld + k0 +
                                                 4 * (lane >> 4));
    }
    static __device__ __forceinline__ floatx4 mma16(short4x a, short4x b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // the same fragments read from an array stored as X[k][m] (m contiguous)
    static __device__ __forceinline__ bf16x8 fragT(const bf16_t* X, int ld, int m0, int k0,
                                                    int lane);
    static __device__ __forceinline__ short4x frag16T(const bf16_t* X, int ld, int m0, int k0,
                                                       int lane);
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    typedef float frag_t;
    typedef float frag16_t;
    // lane l reads one k at row (l % 16), k offset (l / 16)
    static __device__ __forceinline__ float frag(const float* base, int ld, int row0, int k0,
                                                 int lane) {
        return base[(row0 + (lane & 15)) * ld + k0 + (lane >> 4)];
    }
    static __device__ __forceinline__ floatx4 mma(float a, float b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ float frag16(const float*, int, int, int, int) {
        return 0.f;
    }
    static __device__ __forceinline__ floatx4 mma16(float, float, floatx4 c) { return c; }
    // the same fragment read from an array stored as X[k][m] (m contiguous)
    static __device__ __forceinline__ float fragT(const float* X, int ld, int m0, int k0,
                                                   int lane) {
        return X[(k0 + (lane >> 4)) * ld + m0 + (lane & 15)];
    }
    static __device__ __forceinline__ float frag16T(const float*, int, int, int, int) {
        return 0.f;
    }
};

// Fragments of an operand stored with the contraction index strided: the LDS
// array holds X[k][m] (m contiguous) and the MFMA wants, for lane l, the values
// X[k0 + 8 (l/16) + 0..7][m0 + l%16].  ds_read_b64_tr_b16 delivers, within each
// group of 16 lanes, element (l % 4) of the 8-byte pieces addressed by lanes
// 4 j + (l % 16) / 4 (j = 0..3); so lane 4 j + p of group g addresses
// X[k0 + 8 g + j][m0 + 4 p .. 4 p + 3] and receives X[k0 + 8 g + j][m0 + l%16].
typedef __attribute__((address_space(3))) short4x lds_short4x;
typedef short short8x __attribute__((ext_vector_type(8)));

__device__ __forceinline__ short4x read_tr16(const bf16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4x*)(p));
}

__device__ __forceinline__ bf16x8 Mma<bf16_t>::fragT(const bf16_t* X, int ld, int m0, int k0,
                                                     int lane) {
    const int g = lane >> 4, j = (lane & 15) >> 2, p = lane & 3;
    const bf16_t* p0 = X + (k0 + 8 * g + j) * ld + m0 + 4 * p;
    const short4x lo = read_tr16(p0);
    const short4x hi = read_tr16(p0 + 4 * ld);
    const short8x v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// 16-deep version: lane l gets X[k0 + 4 (l/16) + 0..3][m0 + l%16]
__device__ __forceinline__ short4x Mma<bf16_t>::frag16T(const bf16_t* X, int ld, int m0,
                                                        int k0, int lane) {
    const int g = lane >> 4, j = (lane & 15) >> 2, p = lane & 3;
    return read_tr16(X + (k0 + 4 * g + j) * ld + m0 + 4 * p);
}

// acc[bm][bn] += A[m0+16bm : +16, k0:k1] * B[n0+16bn : +16, k0:k1]^T for a BM x BN
// block of 16x16 tiles; both operands row-major with k contiguous, k1 - k0 a
// multiple of 16.  Each fragment read from LDS feeds BN (or BM) instructions.
// AT / BT: the A (B) operand is stored k-major (X[k][m]) and read with
// transposing LDS reads instead of as row-major [m][k].
template <typename E, int BM, int BN, bool AT = false, bool BT = false>
__device__ __forceinline__ void mma_block(floatx4 (&acc)[BM][BN], const E* A, int lda, int m0,
                                          const E* B, int ldb, int n0, int k0, int k1,
                                          int lane) {
    using M = Mma<E>;
    int k = k0;
    for (; k + M::KS <= k1; k += M::KS) {
        typename M::frag_t fa[BM], fb[BN];
#pragma unroll
        for (int i = 0; i < BM; ++i) {
            if constexpr (AT) fa[i] = M::fragT(A, lda, m0 + 16 * i, k, lane);
            else fa[i] = M::frag(A, lda, m0 + 16 * i, k, lane);
        }
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            if constexpr (BT) fb[j] = M::fragT(B, ldb, n0 + 16 * j, k, lane);
            else fb[j] = M::frag(B, ldb, n0 + 16 * j, k, lane);
        }
#pragma unroll
        for (int i = 0; i < BM; ++i)
#pragma unroll
            for (int j = 0; j < BN; ++j) acc[i][j] = M::mma(fa[i], fb[j], acc[i][j]);
    }
    if constexpr (M::KS > 16) {
        if (k < k1) {
            typename M::frag16_t fa[BM], fb[BN];
#pragma unroll
            for (int i = 0; i < BM; ++i) {
                if constexpr (AT) fa[i] = M::frag16T(A, lda, m0 + 16 * i, k, lane);
                else fa[i] = M::frag16(A, lda, m0 + 16 * i, k, lane);
            }
#pragma unroll
            for (int j = 0; j < BN; ++j) {
                if constexpr (BT) fb[j] = M::frag16T(B, ldb, n0 + 16 * j, k, lane);
                else fb[j] = M::frag16(B, ldb, n0 + 16 * j, k, lane);
            }
#pragma unroll
            for (int i = 0; i < BM; ++i)
#pragma unroll
                for (int j = 0; j < BN; ++j) acc[i][j] = M::mma16(fa[i], fb[j], acc[i][j]);
        }
    }
}

// acc += A[m0:m0+16, k0:k1] * B[n0:n0+16, k0:k1]^T  (a single tile)
template <typename E>
__device__ __forceinline__ floatx4 mma_tile(floatx4 acc, const E* A, int lda, int m0,
                                            const E* B, int ldb, int n0, int k0, int k1,
                                            int lane) {
    floatx4 a[1][1] = {{acc}};
    mma_block<E, 1, 1>(a, A, lda, m0, B, ldb, n0, k0, k1, lane);
    return a[0][0];
}

// element e of a 16x16 C tile held by `lane`: row / column inside the tile
__device__ __forceinline__ int c_row(int lane, int e) { return 4 * (lane >> 4) + e; }
__device__ __forceinline__ int c_col(int lane) { return lane & 15; }



// N consecutive elements <-> floats (one 4-byte access for a bf16 pair)
template <typename E, int N>
__device__ __forceinline__ void load_dims(const E* p, float (&x)[N]) {
    if constexpr (N == 2 && sizeof(E) == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xFFFF0000u);
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) x[j] = to_f<E>(p[j]);
    }
}
template <typename E, int N> __device__ __forceinline__ void store_dims(E* p, const E (&x)[N]) {
    if constexpr (N * sizeof(E) == 4) {
        *reinterpret_cast<uint32_t*>(p) = __builtin_bit_cast(uint32_t, x);
    } else if constexpr (N * sizeof(E) == 8) {
        *reinterpret_cast<uint2*>(p) = __builtin_bit_cast(uint2, x);
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) p[j] = x[j];
    }
}

// ------------------------------------------------------------ Moebius maps
// The precision recurrence lambda_t = M_t<lambda_{t-1}> with M<x> = (m11 x +
// m12) / (m21 x + m22) and the token matrix M_t = [[1 + b nu, b a^2], [nu, a^2]]
// ("Kalman Delta Networks" summary, Moebius-transformation structure of the
// precision update); maps compose by matrix product.  Entries are non-negative.
struct M2 {
    float a, b, c, d;  // [[a b] [c d]]
};

__device__ __forceinline__ M2 mob_mul(const M2& x, const M2& y) {
    return {x.a * y.a + x.b * y.c, x.a * y.b + x.b * y.d, x.c * y.a + x.d * y.c,
            x.c * y.b + x.d * y.d};
}

// scale by the power of two that brings the largest entry into [0.5, 1)
__device__ __forceinline__ M2 mob_renorm(const M2& m) {
    const float mx = fmaxf(fmaxf(m.a, m.b), fmaxf(m.c, m.d));
    int e;
    frexpf(mx, &e);
    return {ldexpf(m.a, -e), ldexpf(m.b, -e), ldexpf(m.c, -e), ldexpf(m.d, -e)};
}

__device__ __forceinline__ float mob_apply(const M2& m, float x) {
    return (m.a * x + m.b) / (m.c * x + m.d);
}

// M_t X for one token: M = U_b P with P = [[1, 0], [nu, a^2]] and U_b = [[1, b],
// [0, 1]], so M X = [[x11 + b y1, x12 + b y2], [y1, y2]] with (y1, y2) =
// nu (x11, x12) + a^2 (x21, x22): six multiply-adds.
__device__ __forceinline__ M2 mob_step(const M2& x, float b, float a2, float nu) {
    const float y1 = fmaf(nu, x.a, a2 * x.c);
    const float y2 = fmaf(nu, x.b, a2 * x.d);
    return {fmaf(b, y1, x.a), fmaf(b, y2, x.b), y1, y2};
}

}  // namespace kdn
