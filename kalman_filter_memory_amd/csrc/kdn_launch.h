// kdn_launch.h -- what the kernel sources share on the launch side
// (internal): the dispatch helper that lets a kernel's own dispatch record
// timing events, and the per-head row/chunk addressing of fixed-length and
// packed batches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "kdn_kernels.h"

namespace kdn {

template <typename F, typename... Args>
inline void launch_k(F kernel, dim3 grid, dim3 block, unsigned shmem, hipStream_t st,
                     Args... args) {
    LaunchTiming& t = launch_timing();
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, t.start, t.stop, 0u, args...);
    t = LaunchTiming{};
}

// The token rows and chunks of one head (or, packed, one (sequence, head)):
// first row, tokens, chunks, and its first entry in the per-chunk arrays (Moebius
// products, T matrices, decays: nc each) and in the chunk-boundary precisions
// (nc + 1 each).
struct Slab {
    size_t row0;
    int T, nc;
    size_t c0, l0;
};
template <bool VL>
__device__ __forceinline__ Slab slab_of(size_t bh, int T, int NC, const Packed& pk) {
    if constexpr (!VL) {
        return Slab{bh * T, T, NC, bh * NC, bh * (size_t)(NC + 1)};
    } else {
        const int s = static_cast<int>(bh / pk.H), h = static_cast<int>(bh % pk.H);
        const int b = pk.cu[s], e = pk.cu[s + 1], c0 = pk.cc[s], c1 = pk.cc[s + 1];
        const int nc = c1 - c0;
        return Slab{(size_t)h * pk.Ttot + b, e - b, nc, (size_t)pk.H * c0 + (size_t)h * nc,
                    (size_t)pk.H * (c0 + s) + (size_t)h * (nc + 1)};
    }
}

}  // namespace kdn
