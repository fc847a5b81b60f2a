// kdn_decode.hip -- one-token recurrent decode step of the KDN layer, in place.
//
// Constant-memory decoding ("Kalman Delta Networks", English abstract): each
// (sequence, head) keeps S (d_v x d_k, fp32) and its precision lambda; one
// token performs predict, gain, projection, write and read-out:
//   lambda^- = lambda / (a^2 + nu lambda);  w = P^- k / (k^T P^- k + r)
//   lambda  <- lambda^- + k.k / r  (diagonal)  |  lambda^- + |k|^2/(d_k r)  (isotropic)
//   row j:  u_j = v_j - a s_j.k;  s_j <- a s_j + u_j w;  o_j = a s_j.q + u_j (w.q)
// The last line is o = S_t q expanded so that S is read once and written once.
//
// The step is bound by HBM traffic: 2 * d_v * d_k * 4 bytes of state per
// (sequence, head) against 6 d_k d_v flops.  One workgroup owns one state;
// each lane streams float4 pieces of S rows (d_k / 4 lanes per row), so a
// wave's load covers whole contiguous rows.  The group of d_k / 4 lanes that
// shares a row holds every key dimension, so each group computes the gain in
// full with shuffles: no LDS, and the only barrier orders the reads of lambda
// before its in-place update.  The gain inputs are loaded before the state
// rows, so waiting for them leaves the rows in flight.
#include <atomic>

#include "kdn_device.h"
#include "kdn_launch.h"

namespace kdn {
namespace {

constexpr int kMaxWaves = 8;

template <int DK, int DV> struct DecCfg {
    static constexpr int LPR = DK / 4;         // lanes per S row (one float4 each)
    static constexpr int RPS = kWave / LPR;    // rows covered by one wave-wide load
    static constexpr int NW = DV / RPS < kMaxWaves ? DV / RPS : kMaxWaves;
    static constexpr int RPW = DV / NW;        // rows per wave
    static constexpr int SLOTS = RPW / RPS;    // wave-wide loads per wave
    static_assert(SLOTS >= 1 && RPW % RPS == 0 && DV % NW == 0, "unsupported tile");
};

// four consecutive elements as floats (one 8-byte access for bf16)
template <typename E> __device__ __forceinline__ float4 load4f(const E* p);
template <> __device__ __forceinline__ float4 load4f<float>(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
template <> __device__ __forceinline__ float4 load4f<bf16_t>(const bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

__device__ __forceinline__ float dot4(const float4& x, const float4& y) {
    return x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
}

// INDEXED (continuous batching): the state of active sequence n lives at cache
// slot slot[n] (S and lam then hold n_slots x H states); a slot outside
// [0, n_slots) marks an idle row, whose workgroup returns at once.
template <typename E, typename G, int DK, int DV, bool DIAG, bool INDEXED>
__global__ __launch_bounds__((DecCfg<DK, DV>::NW * kWave)) void decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const G* __restrict__ a, const G* __restrict__ nu, const G* __restrict__ r,
    float* __restrict__ S, float* __restrict__ lam, E* __restrict__ o,
    const int32_t* __restrict__ slot, int H, int n_slots) {
    using Cfg = DecCfg<DK, DV>;
    constexpr int LPR = Cfg::LPR, RPS = Cfg::RPS, RPW = Cfg::RPW, SLOTS = Cfg::SLOTS;

    const size_t st = blockIdx.x;  // (sequence, head) index of the active batch
    size_t sc = st;                // index of its state
    if constexpr (INDEXED) {
        const int sl = slot[st / H];
        if (sl < 0 || sl >= n_slots) return;  // idle row (the whole workgroup)
        sc = (size_t)sl * H + st % H;
    }
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int col = 4 * (lane % LPR), rsub = lane / LPR;

    // ---- gain inputs and values, then the state rows ----
    const float at = to_f<G>(a[st]), nut = to_f<G>(nu[st]), rt = to_f<G>(r[st]);
    const float4 k4 = load4f<E>(k + st * DK + col);
    const float4 q4 = load4f<E>(q + st * DK + col);
    float4 l4;
    if constexpr (DIAG) l4 = *reinterpret_cast<const float4*>(lam + sc * DK + col);
    else l4.x = lam[sc];

    float* Sst = S + sc * (size_t)(DV * DK);
    float4 srow[SLOTS];
    float vj[SLOTS];
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) vj[m] = to_f<E>(v[st * DV + wave * RPW + m * RPS + rsub]);
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
        const int row = wave * RPW + m * RPS + rsub;
        srow[m] = *reinterpret_cast<const float4*>(Sst + row * DK + col);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the row loads ahead of the gain arithmetic

    // ---- predict, gain and projection ----
    const float a2 = at * at;
    float4 w4, ln4;
    if constexpr (DIAG) {
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w};
        float lm[4], pk[4], part = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float dn = a2 + nut * lv[i];
            lm[i] = lv[i] / dn;
            pk[i] = dn / lv[i] * kv[i];  // P^- k
            part += kv[i] * pk[i];
        }
        const float iden = 1.f / (rt + group_sum<LPR>(part)), ir = 1.f / rt;
        w4 = make_float4(pk[0] * iden, pk[1] * iden, pk[2] * iden, pk[3] * iden);
        ln4 = make_float4(lm[0] + kv[0] * kv[0] * ir, lm[1] + kv[1] * kv[1] * ir,
                          lm[2] + kv[2] * kv[2] * ir, lm[3] + kv[3] * kv[3] * ir);
    } else {
        const float kk = group_sum<LPR>(dot4(k4, k4));
        const float lm = l4.x / (a2 + nut * l4.x);
        const float g = 1.f / (kk + rt * lm);
        w4 = make_float4(k4.x * g, k4.y * g, k4.z * g, k4.w * g);
        ln4.x = lm + kk / (static_cast<float>(DK) * rt);
    }
    const float wq = group_sum<LPR>(dot4(w4, q4));
    __syncthreads();  // every wave has read lambda before it is overwritten
    if (wave == 0 && rsub == 0) {
        if constexpr (DIAG) *reinterpret_cast<float4*>(lam + sc * DK + col) = ln4;
        else if (col == 0) lam[sc] = ln4.x;
    }

    // ---- one pass over the rows of S ----
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
        const int row = wave * RPW + m * RPS + rsub;
        const float pk = group_sum<LPR>(dot4(srow[m], k4));
        const float pq = group_sum<LPR>(dot4(srow[m], q4));
        const float u = vj[m] - at * pk;
        float4 ns;
        ns.x = at * srow[m].x + u * w4.x;
        ns.y = at * srow[m].y + u * w4.y;
        ns.z = at * srow[m].z + u * w4.z;
        ns.w = at * srow[m].w + u * w4.w;
        *reinterpret_cast<float4*>(Sst + row * DK + col) = ns;
        if (col == 0) o[st * DV + row] = from_f<E>(at * pq + u * wq);
    }
}

// Compute units of the current device (queried once per device).
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The step is bound by HBM and its workgroups run in rounds of (CUs x
// workgroups per CU).  A last round that is mostly empty keeps too few bytes in
// flight to use the bandwidth, so the workgroups per CU are chosen between the
// three that fit (registers) and two (capped by reserving LDS the kernel does
// not use) by which leaves the fuller last round: 4,096 states on 256 CUs run
// as 8 full rounds of 512 instead of 5 1/3 rounds of 768 (80.2 against 82.0 us).
template <int DK, int DV> unsigned decode_lds_cap(int n_wg) {
    if (DecCfg<DK, DV>::NW != kMaxWaves || n_wg <= 0) return 0;
    const int cus = device_cus();
    auto fill = [&](int per_cu) {  // how full the last round is, in (0, 1]
        const int slots = cus * per_cu;
        const int rem = n_wg % slots;
        return rem == 0 ? 1.0 : static_cast<double>(rem) / slots;
    };
    return fill(2) > fill(3) ? (64u << 10) : 0u;
}

template <typename E, typename G, int DK, int DV>
hipError_t launch_t(const Shape& s, const void* q, const void* k, const void* v, const void* a,
                    const void* nu, const void* r, float* S, float* lam, void* o,
                    const int32_t* slot, int H, int n_slots, hipStream_t st) {
    const dim3 grid(s.BH), block(DecCfg<DK, DV>::NW * kWave);
    const unsigned lds = decode_lds_cap<DK, DV>(s.BH);
    const E* qe = static_cast<const E*>(q);
    const E* ke = static_cast<const E*>(k);
    const E* ve = static_cast<const E*>(v);
    const G* ag = static_cast<const G*>(a);
    const G* ng = static_cast<const G*>(nu);
    const G* rg = static_cast<const G*>(r);
    E* oe = static_cast<E*>(o);
#define KDN_DEC_L(DIAG_, IDX_)                                                             \
    hipLaunchKernelGGL((decode_kernel<E, G, DK, DV, DIAG_, IDX_>), grid, block, lds, st, qe, ke, \
                       ve, ag, ng, rg, S, lam, oe, slot, H, n_slots)
    if (slot) {
        if (s.diag) KDN_DEC_L(true, true);
        else KDN_DEC_L(false, true);
    } else {
        if (s.diag) KDN_DEC_L(true, false);
        else KDN_DEC_L(false, false);
    }
#undef KDN_DEC_L
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const Shape& s, const void* q, const void* k, const void* v, const void* a,
                    const void* nu, const void* r, float* S, float* lam, void* o,
                    const int32_t* slot, int H, int n_slots, hipStream_t st) {
#define KDN_DEC_CASE(DK_, DV_)                                                                \
    if (s.dk == DK_ && s.dv == DV_)                                                           \
        return s.gate_bf16 ? launch_t<E, bf16_t, DK_, DV_>(s, q, k, v, a, nu, r, S, lam, o,   \
                                                           slot, H, n_slots, st)              \
                           : launch_t<E, float, DK_, DV_>(s, q, k, v, a, nu, r, S, lam, o,    \
                                                          slot, H, n_slots, st);
    KDN_DEC_CASE(32, 32) KDN_DEC_CASE(32, 64) KDN_DEC_CASE(32, 128)
    KDN_DEC_CASE(64, 32) KDN_DEC_CASE(64, 64) KDN_DEC_CASE(64, 128)
    KDN_DEC_CASE(128, 32) KDN_DEC_CASE(128, 64) KDN_DEC_CASE(128, 128)
#undef KDN_DEC_CASE
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(const Shape& s) {
    auto ok = [](int d) { return d == 32 || d == 64 || d == 128; };
    return ok(s.dk) && ok(s.dv);
}

hipError_t launch_decode(const Shape& s, const void* q, const void* k, const void* v,
                         const void* a, const void* nu, const void* r, float* S, float* lam,
                         void* o, hipStream_t st, const int32_t* slot, int H, int n_slots) {
    if (s.BH == 0) return hipSuccess;
    return s.qkv_bf16 ? launch_e<bf16_t>(s, q, k, v, a, nu, r, S, lam, o, slot, H, n_slots, st)
                      : launch_e<float>(s, q, k, v, a, nu, r, S, lam, o, slot, H, n_slots, st);
}

}  // namespace kdn
