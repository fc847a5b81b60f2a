// kdn_scan.hip -- the precision (uncertainty) recurrence of the KDN layer as an
// associative scan of 2x2 Moebius matrices, and the Kalman gain.
//
// Per token and per key dimension i (diagonal) or per head (isotropic), with
// evidence b = k_i^2 / r (diagonal) or |k|^2 / (d_k r) (isotropic):
//   lambda_t = (lambda^-_t + b),  lambda^-_t = lambda_{t-1} / (a^2 + nu lambda_{t-1})
// which is the Moebius map of M_t = [[1 + b nu, b a^2], [nu, a^2]]
// ("Kalman Delta Networks", English abstract: because each precision update is
// a linear-fractional map, the whole sequence of them composes associatively
// and can be evaluated by a scan of depth log T).
// A Moebius map does not change when its matrix is scaled, so products are
// renormalised by exact powers of two to stay inside the float range.
//
// Three passes (reduce, carry, emit):
//   reduce: one wave per chunk of `chunk` tokens forms the chunk's matrix
//           product (diagonal: lane = key dimension, sequential over tokens;
//           isotropic: lane = token, ordered wave-wide tree product);
//   carry:  lanes over (segment of chunks, scan): segment products, a
//           log-depth scan of them across lanes, then each lane's walk over
//           its segment, writing the precision at every chunk boundary and
//           lambda_T;
//   emit:   one wave per chunk replays its tokens from the boundary value and
//           writes every predictive precision lambda^-.
// The gain kernel forms w = P^- k / (k^T P^- k + r) from given lambda^-.
#include "kdn_device.h"
#include "kdn_launch.h"

namespace kdn {
namespace {

constexpr int kWavesPerBlock = 4;

__device__ __forceinline__ M2 shfl_down_m2(const M2& m, int off) {
    return {__shfl_down(m.a, off, kWave), __shfl_down(m.b, off, kWave),
            __shfl_down(m.c, off, kWave), __shfl_down(m.d, off, kWave)};
}
__device__ __forceinline__ M2 shfl_up_m2(const M2& m, int off) {
    return {__shfl_up(m.a, off, kWave), __shfl_up(m.b, off, kWave), __shfl_up(m.c, off, kWave),
            __shfl_up(m.d, off, kWave)};
}

__device__ __forceinline__ M2 token_matrix(float b, float a2, float nu) {
    return {1.f + b * nu, b * a2, nu, a2};
}

// key dimensions handled by one lane in the diagonal kernels
template <int DK> struct Lanes {
    static constexpr int IPL = DK >= 64 ? DK / 64 : 1;  // consecutive dims per lane
    static constexpr int ACTIVE = DK / IPL;             // active lanes
};


// ------------------------------------------------------------------ reduce
// one chunk per wave, lanes over key dims; per-token scalars are computed once
// by lane t and broadcast through scalar registers
// The IPL consecutive key elements of one lane as loaded (widened when used,
// so that every load of a chunk can be in flight before the first is needed).
template <typename E, int IPL> struct KeyRaw;
template <> struct KeyRaw<bf16_t, 2> {
    typedef uint32_t type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t rs, unsigned voff,
                                                unsigned soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
    }
    static __device__ __forceinline__ void widen(type u, float (&x)[2]) {
        x[0] = __uint_as_float(u << 16);
        x[1] = __uint_as_float(u & 0xFFFF0000u);
    }
};
template <> struct KeyRaw<bf16_t, 1> {
    typedef uint16_t type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t rs, unsigned voff,
                                                unsigned soff) {
        return __builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0);
    }
    static __device__ __forceinline__ void widen(type u, float (&x)[1]) { x[0] = bf2f(u); }
};
template <> struct KeyRaw<float, 2> {
    typedef unsigned int type __attribute__((ext_vector_type(2)));
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t rs, unsigned voff,
                                                unsigned soff) {
        return __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0);
    }
    static __device__ __forceinline__ void widen(type u, float (&x)[2]) {
        x[0] = __uint_as_float(u[0]);
        x[1] = __uint_as_float(u[1]);
    }
};
template <> struct KeyRaw<float, 1> {
    typedef uint32_t type;
    static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t rs, unsigned voff,
                                                unsigned soff) {
        return __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
    }
    static __device__ __forceinline__ void widen(type u, float (&x)[1]) {
        x[0] = __uint_as_float(u);
    }
};

// one gate value through a buffer resource
template <typename G> struct GateRaw;
template <> struct GateRaw<bf16_t> {
    static __device__ __forceinline__ bf16_t load(__amdgpu_buffer_rsrc_t rs, unsigned off) {
        return __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
    }
};
template <> struct GateRaw<float> {
    static __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t rs, unsigned off) {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
    }
};

// A chunk of 64 tokens is split over two waves of a workgroup (32 keys in
// registers each, eight waves per SIMD); the second wave multiplies the first
// one's product in through LDS.  Besides the chunk's product the kernel stores
// the prefix products after every 16 tokens (agg_subs per chunk): a wave
// records its running product at its 16th token, and the second wave of a
// chunk multiplies the first wave's product into that one too.
template <int C> struct RedSplit {
    static constexpr int SPLIT = C >= 64 ? 2 : 1;       // waves per chunk
    static constexpr int TPW = C / SPLIT;               // tokens per wave
    static constexpr int CPB = kWavesPerBlock / SPLIT;  // chunks per workgroup
};

template <typename E, typename G, int DK, int C, bool VL>
__global__ __launch_bounds__(64 * kWavesPerBlock) void reduce_diag_kernel(
    const E* __restrict__ k, const G* __restrict__ a, const G* __restrict__ nu,
    const G* __restrict__ r, int T, int NC, float4* __restrict__ agg, Packed pk) {
    using L = Lanes<DK>;
    using KR = KeyRaw<E, L::IPL>;
    using RS = RedSplit<C>;
    constexpr int TPW = RS::TPW;
    __shared__ float4 sgate[kWavesPerBlock][TPW];  // per token of the wave: a^2, nu, 1/r
    __shared__ float4 spart[RS::SPLIT > 1 ? RS::CPB : 1][RS::SPLIT > 1 ? DK : 1];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int part = wave % RS::SPLIT, cb = wave / RS::SPLIT;
    const Slab sl = slab_of<VL>(blockIdx.y, T, NC, pk);
    // (packed: a workgroup wholly past its sequence's chunks returns at once)
    if (VL && (int)blockIdx.x * RS::CPB >= sl.nc) return;
    const int c_raw = blockIdx.x * RS::CPB + cb;
    const bool live = c_raw < sl.nc;  // no early exit: the halves of a chunk meet at a barrier
    const int c = live ? c_raw : sl.nc - 1;
    const int t0 = c * C, n = min(C, sl.T - t0);
    const int tb = part * TPW;  // first token of this wave in the chunk
    const bool act = lane < L::ACTIVE;
    // every load first: the gates of token tb + lane, then the keys of the
    // wave's tokens for this lane's dims (rows past the end repeat the last
    // one); row offsets are uniform, only the lane's column varies
    const size_t row0 = sl.row0 + t0;
    const unsigned gbytes = static_cast<unsigned>(n * sizeof(G));
    const unsigned goff = static_cast<unsigned>(min(tb + lane, n - 1) * sizeof(G));
    const G ra = GateRaw<G>::load(buffer_rsrc(a + row0, gbytes), goff);
    const G rnu = GateRaw<G>::load(buffer_rsrc(nu + row0, gbytes), goff);
    const G rr = GateRaw<G>::load(buffer_rsrc(r + row0, gbytes), goff);
    const __amdgpu_buffer_rsrc_t kc =
        buffer_rsrc(k + row0 * DK, static_cast<unsigned>(n * DK * sizeof(E)));
    const unsigned col = (act ? lane : 0) * L::IPL * sizeof(E);
    typename KR::type kr[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u)
        kr[u] = KR::load(kc, col, min(tb + u, n - 1) * DK * sizeof(E));
    // lane t: gates of token tb + t (padding: the identity, a = 1, nu = 0,
    // 1/r = 0), handed to every lane of the wave through LDS (one broadcast read
    // per token).  Padding by arithmetic, not a select, which would be compiled
    // to a branch around the gate loads, placing them after the keys.
    {
        const float at = to_f<G>(ra), m = tb + lane < n ? 1.f : 0.f;
        const float4 g = make_float4(fmaf(at * at, m, 1.f - m), to_f<G>(rnu) * m,
                                     __builtin_amdgcn_rcpf(to_f<G>(rr)) * m, 0.f);
        if (lane < TPW) sgate[wave][lane] = g;
    }
    __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in order
    constexpr int NS = C / 16;  // products kept per (chunk, dim)
    float4* dst = agg + (size_t)(sl.c0 + c) * NS * DK + lane * L::IPL;
    auto put = [&](int s_, int j, const M2& m) {
        if (act && live) {
            const M2 q = mob_renorm(m);
            dst[(size_t)s_ * DK + j] = make_float4(q.a, q.b, q.c, q.d);
        }
    };
    M2 P[L::IPL], mid[L::IPL];
#pragma unroll
    for (int j = 0; j < L::IPL; ++j) P[j] = {1.f, 0.f, 0.f, 1.f};
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        float kv[L::IPL];
        KR::widen(kr[t], kv);
        const float4 g = sgate[wave][t];
#pragma unroll
        for (int j = 0; j < L::IPL; ++j) P[j] = mob_step(P[j], kv[j] * kv[j] * g.z, g.x, g.y);
        if ((t & 7) == 7)
#pragma unroll
            for (int j = 0; j < L::IPL; ++j) P[j] = mob_renorm(P[j]);
        if (t == 15 && TPW > 16)  // the wave's first 16 tokens
#pragma unroll
            for (int j = 0; j < L::IPL; ++j) mid[j] = P[j];
    }
    // the prefix after the first 16 tokens of the chunk (wave 0 of a chunk)
    if (part == 0 && TPW > 16)
#pragma unroll
        for (int j = 0; j < L::IPL; ++j) put(0, j, mid[j]);
    if constexpr (RS::SPLIT > 1) {
        static_assert(RS::SPLIT == 2, "two waves per chunk");
        if (part == 0 && act) {
#pragma unroll
            for (int j = 0; j < L::IPL; ++j) {
                spart[cb][lane * L::IPL + j] = make_float4(P[j].a, P[j].b, P[j].c, P[j].d);
                put(1, j, P[j]);  // the prefix after 32 tokens
            }
        }
        __syncthreads();
        if (part == 0) return;
        if (act) {
#pragma unroll
            for (int j = 0; j < L::IPL; ++j) {
                const float4 f = spart[cb][lane * L::IPL + j];
                const M2 first = {f.x, f.y, f.z, f.w};
                put(2, j, mob_mul(mid[j], first));  // the prefix after 48 tokens
                P[j] = mob_mul(P[j], first);
            }
        }
    }
    {
#pragma unroll
        for (int j = 0; j < L::IPL; ++j) put(NS - 1, j, P[j]);  // the chunk's product
    }
}

// |k_t|^2 of a chunk's tokens (n <= 64 rows from k0), token t's value
// returned in lane t: 16 lanes read each key row in contiguous pieces (one
// vector load of d_k/16 elements per lane), add them with DPP over their row
// of 16 lanes, and hand the sum to the token's lane through the wave's LDS
// slice `sq` (written and read by this wave only, in order).
template <typename E, int DK, int C = 64>
__device__ __forceinline__ float chunk_row_sq(const E* __restrict__ k0, int n, int lane,
                                              float* sq) {
    constexpr int EPL = DK / 16, IT = (C + 3) / 4;
    const int g = lane >> 4, l16 = lane & 15;
    // every row load is issued before the first is used (rows past the end
    // reload the last one; their sums are not stored)
    float x[IT][EPL];
#pragma unroll
    for (int it = 0; it < IT; ++it)
        load_vec<E, EPL>(k0 + size_t(min(g + 4 * it, n - 1)) * DK + l16 * EPL, x[it]);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) s = fmaf(x[it][i], x[it][i], s);
        s = group_sum<16>(s);
        const int t = g + 4 * it;
        if (l16 == 0 && t < n) sq[t] = s;
    }
    // the stores above and the read below are by different lanes of this
    // wave: keep the compiler from moving the read ahead of the stores
    __builtin_amdgcn_wave_barrier();
    return lane < n ? sq[lane] : 0.f;
}

template <typename E, int DK, int C, bool VL>
__global__ __launch_bounds__(64 * kWavesPerBlock) void reduce_iso_kernel(
    const E* __restrict__ k, const void* __restrict__ a, const void* __restrict__ nu,
    const void* __restrict__ r, bool gate_bf16, int T, int NC, float4* __restrict__ agg,
    Packed pk) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int c = blockIdx.x * kWavesPerBlock + wave;
    const Slab sl = slab_of<VL>(blockIdx.y, T, NC, pk);
    if (c >= sl.nc) return;
    const int t0 = c * C, n = min(C, sl.T - t0);
    // the gates first, so that their loads fly with the key rows'
    const size_t tok = sl.row0 + t0 + min(lane, n - 1);
    const float at = load_gate(a, tok, gate_bf16), nut = load_gate(nu, tok, gate_bf16);
    const float rt = load_gate(r, tok, gate_bf16);
    __shared__ float sq[kWavesPerBlock][kWave];
    const float kk = chunk_row_sq<E, DK, C>(k + (sl.row0 + t0) * DK, n, lane, sq[wave]);
    M2 P = {1.f, 0.f, 0.f, 1.f};
    if (lane < n) {
        const float b = kk / (static_cast<float>(DK) * rt);
        P = token_matrix(b, at * at, nut);
    }
    // ordered tree product: later tokens multiply on the left
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const M2 o = shfl_down_m2(P, off);
        if ((lane & (2 * off - 1)) == 0) P = mob_renorm(mob_mul(o, P));
    }
    if (lane == 0) agg[sl.c0 + c] = make_float4(P.a, P.b, P.c, P.d);
}

// ------------------------------------------------------------------- carry
// Each scan (one per (head, key dim) or per head) runs over the chunk maps in
// order.  A wave takes 64 / SEG scans and cuts each into SEG segments of
// consecutive chunks, one lane per (segment, scan): rows of 64 / SEG lanes are
// segments, so the lanes of a row read neighbouring scans' maps together.  A
// lane composes its segment's maps; the segment products are then scanned
// across the rows of lanes in log2(SEG) steps (Hillis-Steele, later segments on
// the left); each lane carries the starting precision through the product of
// the segments before its own and walks its segment writing the precision at
// each chunk start.  Segments of up to kCarryGroup chunks stay in registers
// between the two passes; longer ones are read twice, kCarryGroup maps at a
// time.  SEG grows with the chunk count (4 at 64 chunks, 64 at 1,024), so that
// long sequences spread over more lanes and waves.
constexpr int kCarryGroup = 16;

__device__ __forceinline__ M2 as_m2(const float4& v) { return {v.x, v.y, v.z, v.w}; }

__device__ __forceinline__ float mob_apply_fast(const float4& m, float x) {
    return fmaf(m.x, x, m.y) * __builtin_amdgcn_rcpf(fmaf(m.z, x, m.w));
}

// agg holds NS products per (chunk, scan), the chunk's own product last.
template <int SEG, bool ONE_GROUP, bool VL>
__global__ __launch_bounds__(kWave) void carry_kernel(const float4* __restrict__ agg,
                                                      const float* __restrict__ lambda0, int BH,
                                                      int NL, int NS, int T, int NC_all,
                                                      float* __restrict__ lam_chunk,
                                                      float* __restrict__ lambda_T, Packed pk) {
    constexpr int SC = kWave / SEG;  // scans per wave
    const int lane = threadIdx.x, seg = lane / SC, sl = lane % SC;
    const size_t n_scan = (size_t)BH * NL;
    const size_t idx = blockIdx.x * (size_t)SC + sl;  // bh * NL + i
    const bool valid = idx < n_scan;
    const size_t id = valid ? idx : n_scan - 1;  // loads of lanes past the end stay in range
    const size_t bh = id / NL, i = id % NL;
    const Slab sb = slab_of<VL>(bh, T, NC_all, pk);
    const int NC = sb.nc;
    const float4* src = agg + (sb.c0 * NS + NS - 1) * NL + i;
    const int SL = (NC + SEG - 1) / SEG;
    const int c0 = min(seg * SL, NC), c1 = min(c0 + SL, NC);  // this lane's chunks [c0, c1)
    auto map_at = [&](int c) { return src[(size_t)min(c, NC - 1) * NS * NL]; };

    // (1) the segment's product, later chunks on the left
    float4 buf[kCarryGroup];
    M2 P = {1.f, 0.f, 0.f, 1.f};
    for (int g = c0; g < c1; g += kCarryGroup) {
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) buf[u] = map_at(g + u);
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) {
            if (g + u < c1) P = mob_mul(as_m2(buf[u]), P);
            if ((u & 7) == 7) P = mob_renorm(P);
        }
        if (ONE_GROUP) break;
    }
    P = mob_renorm(P);
    // (2) inclusive scan of the segment products over the segments of a scan
    // (lane seg then holds segments seg..0), then the exclusive one: the
    // product of the segments before this lane's
#pragma unroll
    for (int off = 1; off < SEG; off <<= 1) {
        const M2 q = shfl_up_m2(P, off * SC);
        if (seg >= off) P = mob_renorm(mob_mul(P, q));
    }
    M2 E = shfl_up_m2(P, SC);
    if (seg == 0) E = M2{1.f, 0.f, 0.f, 1.f};
    float lam = lambda0 ? lambda0[id] : 1.f;
    lam = mob_apply_fast(make_float4(E.a, E.b, E.c, E.d), lam);
    // (3) walk the segment
    float* out = lam_chunk ? lam_chunk + sb.l0 * NL + i : nullptr;
    for (int g = c0; g < c1; g += kCarryGroup) {
        if (!ONE_GROUP) {
#pragma unroll
            for (int u = 0; u < kCarryGroup; ++u) buf[u] = map_at(g + u);
        }
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) {
            if (g + u < c1) {
                if (out && valid) out[(size_t)(g + u) * NL] = lam;
                lam = mob_apply_fast(buf[u], lam);
            }
        }
        if (ONE_GROUP) break;
    }
    if (seg == SEG - 1 && valid) {  // the last segment ends at chunk NC
        if (out) out[(size_t)NC * NL] = lam;
        if (lambda_T) lambda_T[id] = lam;
    }
}

// The carry of a diagonal head over many chunks: one workgroup of
// kWideWaves waves takes 16 neighbouring key dimensions of one head; lane l
// holds dimension l % 16 of segment 4 w + l / 16 (w the wave), so the head's
// chunks are cut into 4 kWideWaves segments and every load and store of a wave
// covers 16 neighbouring dimensions (64 contiguous bytes per segment).  The
// segment products are scanned inside a wave (2 steps over its 4 segments) and
// across the waves through LDS (each wave composes the totals of the waves
// before it), then each lane walks its segment.
constexpr int kWideWaves = 16, kWideSeg = 4 * kWideWaves;

__global__ __launch_bounds__(kWave * kWideWaves) void carry_wide_kernel(
    const float4* __restrict__ agg, const float* __restrict__ lambda0, int NL, int NS, int NC,
    float* __restrict__ lam_chunk, float* __restrict__ lambda_T) {
    __shared__ float4 tot[kWideWaves][16];
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int sl = lane & 15, seg = wave * 4 + (lane >> 4);
    const size_t id = blockIdx.x * (size_t)16 + sl;  // bh * NL + i (NL a multiple of 16)
    const size_t bh = id / NL, i = id % NL;
    const float4* src = agg + (bh * (size_t)NC * NS + NS - 1) * NL + i;
    const int SL = (NC + kWideSeg - 1) / kWideSeg;
    const int c0 = min(seg * SL, NC), c1 = min(c0 + SL, NC);
    auto map_at = [&](int c) { return src[(size_t)min(c, NC - 1) * NS * NL]; };

    // (1) the segment's product, later chunks on the left
    float4 buf[kCarryGroup];
    M2 P = {1.f, 0.f, 0.f, 1.f};
    for (int g = c0; g < c1; g += kCarryGroup) {
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) buf[u] = map_at(g + u);
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) {
            if (g + u < c1) P = mob_mul(as_m2(buf[u]), P);
            if ((u & 7) == 7) P = mob_renorm(P);
        }
    }
    P = mob_renorm(P);
    // (2) inclusive scan over the wave's four segments, the wave's total to LDS
#pragma unroll
    for (int off = 16; off < kWave; off <<= 1) {
        const M2 q = shfl_up_m2(P, off);
        if (lane >= off) P = mob_renorm(mob_mul(P, q));
    }
    if (lane >= 48) tot[wave][sl] = make_float4(P.a, P.b, P.c, P.d);
    M2 E = shfl_up_m2(P, 16);  // the segments before this lane's within the wave
    if (lane < 16) E = M2{1.f, 0.f, 0.f, 1.f};
    __syncthreads();
    // (3) the totals of the waves before this one, later waves on the left
    M2 W = {1.f, 0.f, 0.f, 1.f};
    for (int w = 0; w < wave; ++w) W = mob_renorm(mob_mul(as_m2(tot[w][sl]), W));
    E = mob_renorm(mob_mul(E, W));
    float lam = lambda0 ? lambda0[id] : 1.f;
    lam = mob_apply_fast(make_float4(E.a, E.b, E.c, E.d), lam);
    // (4) walk the segment
    float* out = lam_chunk ? lam_chunk + bh * (size_t)(NC + 1) * NL + i : nullptr;
    for (int g = c0; g < c1; g += kCarryGroup) {
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) buf[u] = map_at(g + u);
#pragma unroll
        for (int u = 0; u < kCarryGroup; ++u) {
            if (g + u < c1) {
                if (out) out[(size_t)(g + u) * NL] = lam;
                lam = mob_apply_fast(buf[u], lam);
            }
        }
    }
    if (seg == kWideSeg - 1) {  // the last segment ends at chunk NC
        if (out) out[(size_t)NC * NL] = lam;
        if (lambda_T) lambda_T[id] = lam;
    }
}

// -------------------------------------------------------------------- emit
template <typename E, int DK>
__global__ __launch_bounds__(64 * kWavesPerBlock) void emit_diag_kernel(
    const E* __restrict__ k, const void* __restrict__ a, const void* __restrict__ nu,
    const void* __restrict__ r, bool gate_bf16, int T, int C, int NC,
    const float* __restrict__ lam_chunk, float* __restrict__ lambda_minus) {
    using L = Lanes<DK>;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int c = blockIdx.x * kWavesPerBlock + wave;
    const size_t bh = blockIdx.y;
    if (c >= NC || lane >= L::ACTIVE) return;
    const int t0 = c * C, n = min(C, T - t0);
    float lam[L::IPL];
#pragma unroll
    for (int j = 0; j < L::IPL; ++j)
        lam[j] = lam_chunk[(bh * (NC + 1) + c) * DK + lane * L::IPL + j];
    for (int t = 0; t < n; ++t) {
        const size_t tok = bh * T + t0 + t;
        const float at = load_gate(a, tok, gate_bf16), nut = load_gate(nu, tok, gate_bf16);
        const float ir = 1.f / load_gate(r, tok, gate_bf16);
        float kv[L::IPL];
        load_dims<E, L::IPL>(k + tok * DK + lane * L::IPL, kv);
#pragma unroll
        for (int j = 0; j < L::IPL; ++j) {
            const float lm = lam[j] / (at * at + nut * lam[j]);
            lambda_minus[tok * DK + lane * L::IPL + j] = lm;
            lam[j] = lm + kv[j] * kv[j] * ir;
        }
    }
}

template <typename E, int DK>
__global__ __launch_bounds__(64 * kWavesPerBlock) void emit_iso_kernel(
    const E* __restrict__ k, const void* __restrict__ a, const void* __restrict__ nu,
    const void* __restrict__ r, bool gate_bf16, int T, int C, int NC,
    const float* __restrict__ lam_chunk, float* __restrict__ lambda_minus) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int c = blockIdx.x * kWavesPerBlock + wave;
    const size_t bh = blockIdx.y;
    if (c >= NC) return;
    const int t0 = c * C, n = min(C, T - t0);
    const float lam0 = lam_chunk[bh * (NC + 1) + c];
    __shared__ float sq[kWavesPerBlock][kWave];
    const float kk = chunk_row_sq<E, DK>(k + (bh * T + t0) * DK, n, lane, sq[wave]);
    M2 P = {1.f, 0.f, 0.f, 1.f};
    float at = 1.f, nut = 0.f;
    if (lane < n) {
        const size_t tok = bh * T + t0 + lane;
        at = load_gate(a, tok, gate_bf16);
        nut = load_gate(nu, tok, gate_bf16);
        const float rt = load_gate(r, tok, gate_bf16);
        const float b = kk / (static_cast<float>(DK) * rt);
        P = token_matrix(b, at * at, nut);
    }
    // inclusive prefix product over the chunk's tokens (Hillis-Steele)
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const M2 o = shfl_up_m2(P, off);
        if (lane >= off) P = mob_renorm(mob_mul(P, o));
    }
    const float lam_incl = mob_apply(P, lam0);
    float lam_prev = __shfl_up(lam_incl, 1, kWave);
    if (lane == 0) lam_prev = lam0;
    if (lane < n) lambda_minus[bh * T + t0 + lane] = lam_prev / (at * at + nut * lam_prev);
}

// -------------------------------------------------------------------- gain
// One wave per 16 tokens; lanes over key dimensions.
constexpr int kGainTokensPerWave = 16;

template <typename E, typename W, int DK>
__global__ __launch_bounds__(64 * kWavesPerBlock) void gain_kernel(
    const E* __restrict__ k, const void* __restrict__ r, bool gate_bf16, bool diag,
    size_t n_tok, const float* __restrict__ lambda_minus, W* __restrict__ w) {
    using L = Lanes<DK>;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const size_t tok0 = (blockIdx.x * (size_t)kWavesPerBlock + wave) * kGainTokensPerWave;
    for (int t = 0; t < kGainTokensPerWave; ++t) {
        const size_t tok = tok0 + t;
        if (tok >= n_tok) return;
        const float rt = load_gate(r, tok, gate_bf16);
        float kv[L::IPL], pk[L::IPL];
        float part = 0.f;
        if (lane < L::ACTIVE) {
            load_dims<E, L::IPL>(k + tok * DK + lane * L::IPL, kv);
#pragma unroll
            for (int j = 0; j < L::IPL; ++j) {
                const float lm = diag ? lambda_minus[tok * DK + lane * L::IPL + j]
                                      : lambda_minus[tok];
                pk[j] = kv[j] / lm;  // P^- k
                part += kv[j] * pk[j];
            }
        }
        const float den = wave_sum(part) + rt;
        if (lane < L::ACTIVE) {
#pragma unroll
            for (int j = 0; j < L::IPL; ++j)
                w[tok * DK + lane * L::IPL + j] = from_f<W>(pk[j] / den);
        }
    }
}

// ---------------------------------------------------------------- launchers
template <typename E>
hipError_t reduce_e(const Shape& s, const void* k, const void* a, const void* nu, const void* r,
                    float* agg, hipStream_t st) {
    const dim3 grid((s.nc + kWavesPerBlock - 1) / kWavesPerBlock, s.BH);
    const dim3 block(64 * kWavesPerBlock);
    float4* g = reinterpret_cast<float4*>(agg);
    const E* kk = static_cast<const E*>(k);
#define KDN_RED_DL(G_, VL_, DK_, C_)                                                          \
    launch_k((reduce_diag_kernel<E, G_, DK_, C_, VL_>), gridd, block, 0, st, kk,                \
             static_cast<const G_*>(a), static_cast<const G_*>(nu), static_cast<const G_*>(r), \
             s.T, s.nc, g, s.pk)
#define KDN_RED_D(DK_, C_)                                                                    \
    if (s.diag && s.dk == DK_ && s.chunk == C_) {                                             \
        constexpr int cpb = RedSplit<C_>::CPB;                                                \
        const dim3 gridd((s.nc + cpb - 1) / cpb, s.BH);                                       \
        if (s.gate_bf16) {                                                                    \
            if (s.varlen) KDN_RED_DL(bf16_t, true, DK_, C_);                                  \
            else KDN_RED_DL(bf16_t, false, DK_, C_);                                          \
        } else {                                                                              \
            if (s.varlen) KDN_RED_DL(float, true, DK_, C_);                                   \
            else KDN_RED_DL(float, false, DK_, C_);                                           \
        }                                                                                     \
        return hipGetLastError();                                                             \
    }
#define KDN_RED_IC(DK_, C_)                                                                   \
    if (!s.diag && s.dk == DK_ && s.chunk == C_) {                                            \
        if (s.varlen)                                                                         \
            launch_k((reduce_iso_kernel<E, DK_, C_, true>), grid, block, 0, st, kk, a, nu, r, \
                     s.gate_bf16, s.T, s.nc, g, s.pk);                                        \
        else                                                                                  \
            launch_k((reduce_iso_kernel<E, DK_, C_, false>), grid, block, 0, st, kk, a, nu,   \
                     r, s.gate_bf16, s.T, s.nc, g, s.pk);                                     \
        return hipGetLastError();                                                             \
    }
#define KDN_RED_I(DK_) KDN_RED_IC(DK_, 16) KDN_RED_IC(DK_, 32) KDN_RED_IC(DK_, 64)
#define KDN_RED_DC(DK_) KDN_RED_D(DK_, 16) KDN_RED_D(DK_, 32) KDN_RED_D(DK_, 64)
    KDN_RED_DC(32) KDN_RED_DC(64) KDN_RED_DC(128)
    KDN_RED_I(32) KDN_RED_I(64) KDN_RED_I(128)
#undef KDN_RED_DC
#undef KDN_RED_I
#undef KDN_RED_IC
#undef KDN_RED_D
#undef KDN_RED_DL
    return hipErrorInvalidValue;
}

template <typename E>
hipError_t emit_e(const Shape& s, const void* k, const void* a, const void* nu, const void* r,
                  const float* lam_chunk, float* lm, hipStream_t st) {
    const dim3 grid((s.nc + kWavesPerBlock - 1) / kWavesPerBlock, s.BH);
    const dim3 block(64 * kWavesPerBlock);
    const E* kk = static_cast<const E*>(k);
#define KDN_EMIT(DK_)                                                                        \
    if (s.dk == DK_) {                                                                       \
        if (s.diag)                                                                          \
            launch_k((emit_diag_kernel<E, DK_>), grid, block, 0, st, kk, a, nu, r,   \
                               s.gate_bf16, s.T, s.chunk, s.nc, lam_chunk, lm);              \
        else                                                                                 \
            launch_k((emit_iso_kernel<E, DK_>), grid, block, 0, st, kk, a, nu, r,    \
                               s.gate_bf16, s.T, s.chunk, s.nc, lam_chunk, lm);              \
        return hipGetLastError();                                                            \
    }
    KDN_EMIT(32) KDN_EMIT(64) KDN_EMIT(128)
#undef KDN_EMIT
    return hipErrorInvalidValue;
}

template <typename E, typename W>
hipError_t gain_ew(const Shape& s, const void* k, const void* r, const float* lm, void* w,
                   hipStream_t st) {
    const size_t n_tok = (size_t)s.BH * s.T;
    const size_t per_block = (size_t)kWavesPerBlock * kGainTokensPerWave;
    const dim3 grid((unsigned)((n_tok + per_block - 1) / per_block));
    const dim3 block(64 * kWavesPerBlock);
    const E* kk = static_cast<const E*>(k);
    W* ww = static_cast<W*>(w);
#define KDN_GAIN(DK_)                                                                      \
    if (s.dk == DK_) {                                                                     \
        launch_k((gain_kernel<E, W, DK_>), grid, block, 0, st, kk, r, s.gate_bf16, \
                           s.diag, n_tok, lm, ww);                                         \
        return hipGetLastError();                                                          \
    }
    KDN_GAIN(32) KDN_GAIN(64) KDN_GAIN(128)
#undef KDN_GAIN
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_scan_reduce(const Shape& s, const void* k, const void* a, const void* nu,
                              const void* r, float* agg, hipStream_t st) {
    if (s.BH == 0 || s.nc == 0) return hipSuccess;
    return s.qkv_bf16 ? reduce_e<bf16_t>(s, k, a, nu, r, agg, st)
                      : reduce_e<float>(s, k, a, nu, r, agg, st);
}

// Offsets of a packed batch: a sanitised copy of the caller's sequence
// offsets (clamped to [0, Ttot] and made non-decreasing, so that every index
// derived from them stays inside the buffers) and the chunk offsets cc.
__global__ void packed_table_kernel(const int32_t* __restrict__ cu_in, int N, int Ttot, int C,
                                    int32_t* __restrict__ cu, int32_t* __restrict__ cc) {
    if (threadIdx.x != 0) return;
    int prev = 0, chunks = 0;
    cu[0] = 0;
    cc[0] = 0;
    for (int s = 0; s < N; ++s) {
        const int e = min(max(cu_in[s + 1], prev), Ttot);
        chunks += (e - prev + C - 1) / C;
        cu[s + 1] = e;
        cc[s + 1] = chunks;
        prev = e;
    }
}

hipError_t launch_packed_table(const int32_t* cu_in, int N, int Ttot, int C, int32_t* cu,
                               int32_t* cc, hipStream_t st) {
    hipLaunchKernelGGL(packed_table_kernel, dim3(1), dim3(64), 0, st, cu_in, N, Ttot, C, cu, cc);
    return hipGetLastError();
}

hipError_t launch_scan_carry(const Shape& s, const float* agg, const float* lambda0,
                             float* lam_chunk, float* lambda_T, hipStream_t st) {
    const int NL = s.diag ? s.dk : 1;
    const size_t n = (size_t)s.BH * NL;
    if (n == 0) return hipSuccess;
    // many chunks and at least 16 key dimensions per head: the wide carry
    if (!s.varlen && NL % 16 == 0 && s.nc > 4 * kCarryGroup) {
        launch_k(carry_wide_kernel, dim3((unsigned)(n / 16)), dim3(kWave * kWideWaves), 0, st,
                 reinterpret_cast<const float4*>(agg), lambda0, NL, agg_subs(s), s.nc, lam_chunk,
                 lambda_T);
        return hipGetLastError();
    }
    // segments per scan: about 16 chunks each, 4 to 64
    int seg = 4;
    while (seg < 64 && seg * kCarryGroup < s.nc) seg *= 2;
    const bool one = s.nc <= seg * kCarryGroup;
    const float4* a4 = reinterpret_cast<const float4*>(agg);
#define KDN_CARRY_L(SEG_, ONE_, VL_)                                                           \
    launch_k(carry_kernel<SEG_, ONE_, VL_>, dim3((unsigned)((n + kWave / SEG_ - 1) / (kWave / SEG_))), \
             dim3(kWave), 0, st, a4, lambda0, s.BH, NL, agg_subs(s), s.T, s.nc, lam_chunk, lambda_T, \
             s.pk)
#define KDN_CARRY_S(SEG_)                                                                      \
    if (seg == SEG_) {                                                                         \
        if (s.varlen) {                                                                        \
            if (one) KDN_CARRY_L(SEG_, true, true);                                            \
            else KDN_CARRY_L(SEG_, false, true);                                               \
        } else {                                                                               \
            if (one) KDN_CARRY_L(SEG_, true, false);                                           \
            else KDN_CARRY_L(SEG_, false, false);                                              \
        }                                                                                      \
    }
    KDN_CARRY_S(4) KDN_CARRY_S(8) KDN_CARRY_S(16) KDN_CARRY_S(32) KDN_CARRY_S(64)
#undef KDN_CARRY_S
#undef KDN_CARRY_L
    return hipGetLastError();
}

hipError_t launch_scan_emit(const Shape& s, const void* k, const void* a, const void* nu,
                            const void* r, const float* lam_chunk, float* lambda_minus,
                            hipStream_t st) {
    if (s.BH == 0 || s.nc == 0) return hipSuccess;
    return s.qkv_bf16 ? emit_e<bf16_t>(s, k, a, nu, r, lam_chunk, lambda_minus, st)
                      : emit_e<float>(s, k, a, nu, r, lam_chunk, lambda_minus, st);
}

hipError_t launch_gain(const Shape& s, const void* k, const void* r, const float* lambda_minus,
                       void* w, hipStream_t st) {
    if (s.BH == 0 || s.T == 0) return hipSuccess;
    if (s.qkv_bf16)
        return s.gain_bf16 ? gain_ew<bf16_t, bf16_t>(s, k, r, lambda_minus, w, st)
                           : gain_ew<bf16_t, float>(s, k, r, lambda_minus, w, st);
    return s.gain_bf16 ? gain_ew<float, bf16_t>(s, k, r, lambda_minus, w, st)
                       : gain_ew<float, float>(s, k, r, lambda_minus, w, st);
}

}  // namespace kdn
