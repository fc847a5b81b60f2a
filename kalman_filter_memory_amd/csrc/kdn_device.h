// kdn_device.h -- device helpers shared by the libkdn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kdn {

typedef uint16_t bf16_t;  // bfloat16 storage
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef short short4x __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16, round to nearest even (inputs are finite).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
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

// fast reciprocal (v_rcp_f32, about 1 ulp)
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ------------------------------------------------------------------- MFMA
// 16x16 output tiles.  Operand fragments are read from row-major LDS arrays
// whose contraction index is contiguous:  A as [m][k], B as [n][k].
// Output (C) layout of one 16x16 tile for lane l:  element e (0..3) holds
// C[4*(l/16) + e][l % 16].
template <typename E> struct Mma;

template <> struct Mma<bf16_t> {
    static constexpr int KS = 32;  // contraction depth of one instruction
    // lane l reads 8 consecutive k at row (l % 16), k offset 8 * (l / 16)
    static __device__ __forceinline__ bf16x8 frag(const bf16_t* base, int ld, int row0, int k0,
                                                  int lane) {
        const bf16_t* p = base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4);
        return *reinterpret_cast<const bf16x8*>(p);
    }
    static __device__ __forceinline__ floatx4 mma(bf16x8 a, bf16x8 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // a 16-deep step (v_mfma_f32_16x16x16_bf16): lane l reads 4 consecutive k
    // at row (l % 16), k offset 4 * (l / 16)
    static __device__ __forceinline__ floatx4 mma16(const bf16_t* A, int lda, int m0,
                                                    const bf16_t* B, int ldb, int n0, int k,
                                                    int lane, floatx4 c) {
        const short4x fa = *reinterpret_cast<const short4x*>(A + (m0 + (lane & 15)) * lda + k +
                                                            4 * (lane >> 4));
        const short4x fb = *reinterpret_cast<const short4x*>(B + (n0 + (lane & 15)) * ldb + k +
                                                            4 * (lane >> 4));
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, c, 0, 0, 0);
    }
    typedef bf16x8 frag_t;
};

template <> struct Mma<float> {
    static constexpr int KS = 4;
    // lane l reads one k at row (l % 16), k offset (l / 16)
    static __device__ __forceinline__ float frag(const float* base, int ld, int row0, int k0,
                                                 int lane) {
        return base[(row0 + (lane & 15)) * ld + k0 + (lane >> 4)];
    }
    static __device__ __forceinline__ floatx4 mma(float a, float b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    typedef float frag_t;
};

// acc += A[m0:m0+16, k0:k1] * B[n0:n0+16, k0:k1]^T  (both row-major, k contiguous;
// k1 - k0 a multiple of 16)
template <typename E>
__device__ __forceinline__ floatx4 mma_tile(floatx4 acc, const E* A, int lda, int m0,
                                            const E* B, int ldb, int n0, int k0, int k1,
                                            int lane) {
    int k = k0;
    for (; k + Mma<E>::KS <= k1; k += Mma<E>::KS) {
        auto fa = Mma<E>::frag(A, lda, m0, k, lane);
        auto fb = Mma<E>::frag(B, ldb, n0, k, lane);
        acc = Mma<E>::mma(fa, fb, acc);
    }
    if constexpr (Mma<E>::KS > 16) {
        if (k < k1) acc = Mma<E>::mma16(A, lda, m0, B, ldb, n0, k, lane, acc);
    }
    return acc;
}

// element e of a 16x16 C tile held by `lane`: row / column inside the tile
__device__ __forceinline__ int c_row(int lane, int e) { return 4 * (lane >> 4) + e; }
__device__ __forceinline__ int c_col(int lane) { return lane & 15; }

}  // namespace kdn
