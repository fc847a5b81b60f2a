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
// (sequence, head) against 6 d_k d_v flops.  One workgroup (4 waves) owns one
// state; each lane streams float4 pieces of S rows (d_k / 4 lanes per row), so
// a wave's load covers whole contiguous rows.
#include "kdn_device.h"
#include "kdn_kernels.h"

namespace kdn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum(float x, float* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    x = wave_sum(x);
    __syncthreads();  // red may still be read by a previous block_sum
    if (lane == 0) red[wave] = x;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

template <typename E, int DK, int DV>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const void* __restrict__ a, const void* __restrict__ nu, const void* __restrict__ r,
    bool gate_bf16, bool diag, float* __restrict__ S, float* __restrict__ lam,
    E* __restrict__ o) {
    constexpr int LPR = DK / 4;            // lanes per S row (one float4 each)
    constexpr int RPS = kWave / LPR;       // rows covered by one wave-wide load
    constexpr int ROWS_PER_WAVE = DV / 4;  // 4 waves share the d_v rows
    constexpr int SLOTS = ROWS_PER_WAVE / RPS;
    static_assert(SLOTS >= 1 && ROWS_PER_WAVE % RPS == 0, "unsupported tile");

    __shared__ float sk[DK], sq[DK], sw[DK];
    __shared__ float red[4];

    const size_t st = blockIdx.x;  // (sequence, head) index
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float at = load_gate(a, st, gate_bf16);
    const float nut = load_gate(nu, st, gate_bf16);
    const float rt = load_gate(r, st, gate_bf16);
    const float a2 = at * at;

    // ---- predict, gain and projection (d_k lanes) ----
    float ki = 0.f, qi = 0.f, li = 0.f;
    if (tid < DK) {
        ki = to_f<E>(k[st * DK + tid]);
        qi = to_f<E>(q[st * DK + tid]);
        li = diag ? lam[st * DK + tid] : lam[st];
    }
    float wi = 0.f;
    if (diag) {
        float lmi = 1.f, pi = 0.f;
        if (tid < DK) {
            lmi = li / (a2 + nut * li);
            pi = 1.f / lmi;
        }
        const float den = rt + block_sum(ki * ki * pi, red);
        if (tid < DK) {
            wi = pi * ki / den;
            lam[st * DK + tid] = lmi + ki * ki / rt;
        }
    } else {
        const float kk = block_sum(ki * ki, red);
        const float lm = li / (a2 + nut * li);
        wi = ki / (kk + rt * lm);
        if (tid == 0) lam[st] = lm + kk / (static_cast<float>(DK) * rt);
    }
    const float wq = block_sum(wi * qi, red);
    if (tid < DK) {
        sk[tid] = ki;
        sq[tid] = qi;
        sw[tid] = wi;
    }
    __syncthreads();

    // ---- one pass over the rows of S ----
    const int col = 4 * (lane % LPR);
    const float4 k4 = make_float4(sk[col], sk[col + 1], sk[col + 2], sk[col + 3]);
    const float4 q4 = make_float4(sq[col], sq[col + 1], sq[col + 2], sq[col + 3]);
    const float4 w4 = make_float4(sw[col], sw[col + 1], sw[col + 2], sw[col + 3]);
    float* Sst = S + st * (size_t)(DV * DK);
    float4 srow[SLOTS];
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
        const int row = wave * ROWS_PER_WAVE + m * RPS + lane / LPR;
        srow[m] = *reinterpret_cast<const float4*>(Sst + row * DK + col);
    }
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
        const int row = wave * ROWS_PER_WAVE + m * RPS + lane / LPR;
        float pk = srow[m].x * k4.x + srow[m].y * k4.y + srow[m].z * k4.z + srow[m].w * k4.w;
        float pq = srow[m].x * q4.x + srow[m].y * q4.y + srow[m].z * q4.z + srow[m].w * q4.w;
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) {
            pk += __shfl_xor(pk, off, kWave);
            pq += __shfl_xor(pq, off, kWave);
        }
        const float vj = to_f<E>(v[st * DV + row]);
        const float u = vj - at * pk;
        float4 ns;
        ns.x = at * srow[m].x + u * w4.x;
        ns.y = at * srow[m].y + u * w4.y;
        ns.z = at * srow[m].z + u * w4.z;
        ns.w = at * srow[m].w + u * w4.w;
        *reinterpret_cast<float4*>(Sst + row * DK + col) = ns;
        if ((lane % LPR) == 0) o[st * DV + row] = from_f<E>(at * pq + u * wq);
    }
}

template <typename E, int DK, int DV>
hipError_t launch_t(const Shape& s, const void* q, const void* k, const void* v, const void* a,
                    const void* nu, const void* r, float* S, float* lam, void* o,
                    hipStream_t st) {
    hipLaunchKernelGGL((decode_kernel<E, DK, DV>), dim3(s.BH), dim3(kThreads), 0, st,
                       static_cast<const E*>(q), static_cast<const E*>(k),
                       static_cast<const E*>(v), a, nu, r, s.gate_bf16, s.diag, S, lam,
                       static_cast<E*>(o));
    return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const Shape& s, const void* q, const void* k, const void* v, const void* a,
                    const void* nu, const void* r, float* S, float* lam, void* o,
                    hipStream_t st) {
#define KDN_DEC_CASE(DK_, DV_)                                                   \
    if (s.dk == DK_ && s.dv == DV_)                                              \
        return launch_t<E, DK_, DV_>(s, q, k, v, a, nu, r, S, lam, o, st);
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
                         void* o, hipStream_t st) {
    if (s.BH == 0) return hipSuccess;
    return s.qkv_bf16 ? launch_e<bf16_t>(s, q, k, v, a, nu, r, S, lam, o, st)
                      : launch_e<float>(s, q, k, v, a, nu, r, S, lam, o, st);
}

}  // namespace kdn
