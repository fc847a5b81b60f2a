// abi_host_driver.cpp -- host-only check of the C ABI's validation and
// workspace layout (kdn_api.cpp), built with a host compiler under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
//
// The kernel launchers are replaced by recording stubs: no GPU is touched and
// no device pointer is dereferenced (the tensors are fake, 256-byte aligned
// addresses).  Each stub checks that every buffer it receives inside the
// caller's workspace lies wholly inside it, and that the buffers written by
// the launches of one call do not overlap.  main() walks the entry points over
// supported and unsupported descriptors and checks the returned statuses.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kdn.h"
#include "kdn_kernels.h"

namespace {

int g_fail = 0;
int g_launches = 0;
int g_seg_packed = 0;  // segmented state passes of packed batches seen
// fake device addresses: tensors far below the workspace, never dereferenced
const uintptr_t kTensorBase = uintptr_t(1) << 40;
const uintptr_t kWsBase = uintptr_t(1) << 44;
uintptr_t g_ws_lo = kWsBase, g_ws_hi = kWsBase;

struct Region {
    uintptr_t lo, hi;
    std::string name;
};
std::vector<Region> g_written;

void fail(const std::string& msg) {
    ++g_fail;
    if (g_fail <= 50) std::fprintf(stderr, "FAIL: %s\n", msg.c_str());
}

size_t esz(bool bf16) { return bf16 ? 2 : 4; }

// a buffer of `bytes` at p: the fake tensors lie below the workspace's base
// address, so anything at or above it is a workspace buffer and must lie
// wholly inside the workspace of the current call
void in_ws(const void* p, size_t bytes, const char* name, bool written) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (!p || bytes == 0) return;
    if (a >= g_ws_lo) {
        if (a + bytes > g_ws_hi)
            fail(std::string(name) + " runs past the end of the workspace by " +
                 std::to_string(a + bytes - g_ws_hi) + " bytes");
        if (a % 16) fail(std::string(name) + " is not 16-byte aligned");
        if (written) {
            for (const Region& r : g_written)
                if (a < r.hi && r.lo < a + bytes && r.name != name)
                    fail(std::string(name) + " overlaps " + r.name);
            g_written.push_back({a, a + bytes, name});
        }
    }
}

size_t nl(const kdn::Shape& s) { return s.diag ? s.dk : 1; }

// per-chunk arrays of a packed batch are sized by the chunk-count bound
size_t chunks(const kdn::Shape& s) {
    if (!s.varlen) return (size_t)s.BH * s.nc;
    const size_t N = s.BH / s.pk.H;
    return (size_t)s.pk.H * ((s.pk.Ttot + N * (s.chunk - 1)) / s.chunk);
}
size_t bounds(const kdn::Shape& s) {  // chunk-boundary entries
    if (!s.varlen) return (size_t)s.BH * (s.nc + 1);
    return chunks(s) + (size_t)s.BH;
}
size_t rows(const kdn::Shape& s) {
    return s.varlen ? (size_t)s.pk.H * s.pk.Ttot : (size_t)s.BH * s.T;
}

int dvt_of(const kdn::Shape& s) {
    if (!s.qkv_bf16 && s.dk == 128 && s.chunk == 64) return 0;
    return s.dv >= 64 ? 64 : 32;
}

}  // namespace

// ------------------------------------------------------------ launcher stubs
namespace kdn {

bool chunk_supported(const Shape& s) {
    auto ok = [](int d) { return d == 32 || d == 64 || d == 128; };
    return ok(s.dk) && ok(s.dv) && (s.chunk == 16 || s.chunk == 32 || s.chunk == 64) &&
           dvt_of(s) > 0;
}
bool decode_supported(const Shape& s) { return s.dk >= 32 && s.dv >= 32; }
bool backward_supported(const Shape& s) { return chunk_supported(s); }

// A stand-in planner (the API only passes its plan through and sizes the
// workspace by it): few units and many chunks give 3 .. 8 segments, the first
// about 1.25 times as long as the others.
SegSplit state_split(const Shape& s) {
    const int dvt = dvt_of(s);
    if (s.BH > 0 && dvt > 0 && s.nc >= 16) {
        const int units = s.BH * (s.dv / dvt);
        if (units < 128) {
            int n = 256 / units;
            if (n > 8) n = 8;
            if (s.nc / 4 < n) n = s.nc / 4;
            if (n >= 3) {
                const int Lc = static_cast<int>((s.nc * 4L + 4L * (n - 1) + 4) / (4L * (n - 1) + 5));
                const int L0 = s.nc - (n - 1) * Lc;
                if (L0 >= 1) return SegSplit{n, Lc, L0};
            }
        }
    }
    return SegSplit{1, s.nc, s.nc};
}

hipError_t launch_scan_reduce(const Shape& s, const void*, const void*, const void*,
                              const void*, float* agg, hipStream_t) {
    ++g_launches;
    in_ws(agg, chunks(s) * agg_subs(s) * nl(s) * 16, "agg", true);
    return hipSuccess;
}
hipError_t launch_packed_table(const int32_t*, int N, int, int, int32_t* cu, int32_t* cc,
                               hipStream_t) {
    ++g_launches;
    in_ws(cu, (size_t)(N + 1) * 4, "cu", true);
    in_ws(cc, (size_t)(N + 1) * 4, "cc", true);
    return hipSuccess;
}
hipError_t launch_scan_carry(const Shape& s, const float* agg, const float*, float* lc,
                             float*, hipStream_t) {
    ++g_launches;
    in_ws(agg, chunks(s) * agg_subs(s) * nl(s) * 16, "agg", false);
    in_ws(lc, bounds(s) * nl(s) * 4, "lam_chunk", true);
    return hipSuccess;
}
hipError_t launch_scan_emit(const Shape& s, const void*, const void*, const void*, const void*,
                            const float* lc, float*, hipStream_t) {
    ++g_launches;
    in_ws(lc, bounds(s) * nl(s) * 4, "lam_chunk", false);
    return hipSuccess;
}
hipError_t launch_gain(const Shape&, const void*, const void*, const float*, void*,
                       hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_chunk_prep(const Shape& s, bool fuse, const void*, const void*, const void*,
                             const void*, const float* lc, const float* agg, void* w, void* Tm,
                             float* g, hipStream_t, float* dinv) {
    ++g_launches;
    if (fuse) {
        if (s.diag && !agg) fail("fused diagonal prep without the scan's products");
        in_ws(agg, chunks(s) * agg_subs(s) * nl(s) * 16, "agg", false);
        in_ws(lc, bounds(s) * nl(s) * 4, "lam_chunk", false);
        in_ws(w, rows(s) * s.dk * esz(s.gain_bf16), "w", true);
    }
    in_ws(Tm, chunks(s) * s.chunk * s.chunk * esz(s.qkv_bf16), "T", true);
    in_ws(g, chunks(s) * s.chunk * 4, "g", true);
    in_ws(dinv, rows(s) * 4, "dinv", true);
    return hipSuccess;
}
hipError_t launch_chunk_state(const Shape& s, const void*, const void*, const void*,
                              const float* g, const void* w, const void* Tm, const float*, void*,
                              float*, hipStream_t, void* Sc, const SegWs* seg) {
    ++g_launches;
    in_ws(g, chunks(s) * s.chunk * 4, "g", false);
    in_ws(w, rows(s) * s.dk * esz(s.qkv_bf16), "w", false);
    in_ws(Tm, chunks(s) * s.chunk * s.chunk * esz(s.qkv_bf16), "T", false);
    in_ws(Sc, chunks(s) * s.dv * s.dk * esz(s.qkv_bf16), "Sc", true);
    if (seg && seg->nseg > 1) {
        const SegSplit sp = state_split(s);
        if (s.varlen) {
            // packed: every slab cuts its own chunks into nseg segments
            ++g_seg_packed;
            if (seg->Lc != 0 || seg->nseg > sp.nseg) fail("packed segment plan");
        } else {
            if (sp.nseg != seg->nseg || sp.Lc != seg->Lc || sp.L0 != seg->L0)
                fail("segment plan differs from state_split");
            if (seg->L0 < 1 || seg->Lc < 1 || seg->L0 + (size_t)(seg->nseg - 1) * seg->Lc != (size_t)s.nc)
                fail("segments do not cover the chunks exactly");
        }
        in_ws(seg->Sseg, (size_t)s.BH * seg->nseg * s.dv * s.dk * 4, "Sseg", true);
        in_ws(seg->Aseg, (size_t)s.BH * seg->nseg * s.dk * s.dk * 4, "Aseg", true);
    }
    return hipSuccess;
}
hipError_t launch_decode(const Shape&, const void*, const void*, const void*, const void*,
                         const void*, const void*, float*, float*, void*, hipStream_t,
                         const int32_t*, int, int) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_bwd_state(const Shape& s, const BwdArgs& b, hipStream_t) {
    ++g_launches;
    in_ws(b.dSe, chunks(s) * s.dv * s.dk * esz(s.qkv_bf16), "dSe", true);
    in_ws(b.Sc, chunks(s) * s.dv * s.dk * esz(s.qkv_bf16), "Sc", false);
    return hipSuccess;
}
hipError_t launch_bwd_grad(const Shape& s, const BwdArgs& b, hipStream_t) {
    ++g_launches;
    in_ws(b.dW, rows(s) * s.dk * esz(s.qkv_bf16), "dW", true);
    in_ws(b.sdot, rows(s) * 4, "sdot", true);
    in_ws(b.dlna, rows(s) * 4, "dlna", true);
    in_ws(b.dinv, rows(s) * 4, "dinv", false);
    return hipSuccess;
}
hipError_t launch_bwd_gain(const Shape& s, const BwdArgs& b, hipStream_t) {
    ++g_launches;
    in_ws(b.ab, chunks(s) * nl(s) * 8, "ab", true);
    in_ws(b.Gout, chunks(s) * nl(s) * 4, "Gout", true);
    return hipSuccess;
}
hipError_t launch_dense_gain(const Shape&, const void*, const void*, const void*, const void*,
                             const float*, void*, float*, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}

}  // namespace kdn

// ------------------------------------------------------------------- driver
namespace {

void* fake(int i) { return reinterpret_cast<void*>(kTensorBase + (uintptr_t(i) << 32)); }

kdn_desc desc(int B, int H, int T, int dk, int dv, int C, int var, int qkv, int gate) {
    kdn_desc d;
    d.B = B;
    d.H = H;
    d.T = T;
    d.d_k = dk;
    d.d_v = dv;
    d.chunk = C;
    d.variant = var;
    d.qkv_dtype = qkv;
    d.gate_dtype = gate;
    d.gain_dtype = qkv;
    return d;
}

void begin_call(size_t ws_bytes) {
    g_ws_lo = kWsBase;
    g_ws_hi = kWsBase + ws_bytes;
    g_written.clear();
}

void expect(kdn_status got, kdn_status want, const std::string& what) {
    if (got != want)
        fail(what + ": status " + std::to_string(got) + ", expected " + std::to_string(want));
}

std::string name(const kdn_desc& d) {
    char b[160];
    std::snprintf(b, sizeof b, "B%d H%d T%d dk%d dv%d C%d var%d qkv%d gate%d", d.B, d.H, d.T,
                  d.d_k, d.d_v, d.chunk, d.variant, d.qkv_dtype, d.gate_dtype);
    return b;
}

void forward_case(const kdn_desc& d) {
    const size_t ws = kdn_forward_workspace_bytes(&d);
    void* W = reinterpret_cast<void*>(kWsBase);
    float* lam = static_cast<float*>(fake(7));
    float* S = static_cast<float*>(fake(8));
    void* events[8] = {};
    begin_call(ws);
    const int before = g_launches;
    expect(kdn_forward_events(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                              fake(6), S, lam, W, ws, nullptr, events),
           KDN_OK, "forward " + name(d));
    if (d.B * d.H > 0 && d.T > 0 && g_launches - before != 4)
        fail("forward launched " + std::to_string(g_launches - before) + " kernels: " + name(d));
    // the timing aid: a range of the forward's kernels, reps passes, outputs
    // apart from the inputs (aliasing ones are refused)
    float* lamT = static_cast<float*>(fake(10));
    float* ST = static_cast<float*>(fake(11));
    begin_call(ws);
    const int before_rep = g_launches;
    expect(kdn_forward_repeat(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                              fake(6), ST, lamT, W, ws, nullptr, 1, 3, 2),
           KDN_OK, "forward repeat " + name(d));
    if (d.B * d.H > 0 && d.T > 0 && g_launches - before_rep != 6)
        fail("forward repeat launched " + std::to_string(g_launches - before_rep) +
             " kernels: " + name(d));
    expect(kdn_forward_repeat(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                              fake(6), S, lamT, W, ws, nullptr, 3, 3, 1),
           KDN_ERR_SHAPE, "forward repeat with S_T aliasing S0 " + name(d));
    begin_call(ws);
    expect(kdn_forward(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                       fake(6), S, lam, W, ws ? ws - 1 : 0, nullptr),
           d.B * d.H == 0 ? KDN_OK : KDN_ERR_WORKSPACE, "short workspace " + name(d));
    if (d.B * d.H > 0 && d.T > 0) {
        expect(kdn_forward(&d, nullptr, fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                           fake(6), S, lam, W, ws, nullptr),
               KDN_ERR_NULL, "null q " + name(d));
        expect(kdn_forward(&d, static_cast<char*>(fake(0)) + 2, fake(1), fake(2), fake(3),
                           fake(4), fake(5), lam, S, fake(6), S, lam, W, ws, nullptr),
               KDN_ERR_ALIGN, "misaligned q " + name(d));
    }
    // the Moebius scan and the given-gain stage call on their own workspaces
    const size_t wss = kdn_mobius_scan_workspace_bytes(&d);
    begin_call(wss);
    expect(kdn_mobius_scan(&d, fake(1), fake(3), fake(4), fake(5), lam, static_cast<float*>(fake(9)),
                           nullptr, lam, W, wss, nullptr),
           KDN_OK, "mobius_scan " + name(d));
    const size_t wsd = kdn_chunk_delta_workspace_bytes(&d);
    begin_call(wsd);
    expect(kdn_chunk_delta(&d, fake(0), fake(1), fake(2), fake(3), fake(10), S, fake(6), S, W, wsd,
                           nullptr),
           KDN_OK, "chunk_delta " + name(d));
    // the backward, self-contained and kept
    const size_t wsb = kdn_backward_workspace_bytes(&d);
    if (wsb) {
        float* g[8];
        for (int i = 0; i < 8; ++i) g[i] = static_cast<float*>(fake(11 + i));
        void* bev[14] = {};
        begin_call(wsb);
        expect(kdn_backward_events(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam,
                                   S, fake(20), S, lam, g[0], g[1], g[2], g[3], g[4], g[5], g[6],
                                   g[7], W, wsb, nullptr, bev),
               KDN_OK, "backward " + name(d));
        begin_call(wsb);
        expect(kdn_forward_keep(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                                fake(6), S, lam, W, wsb, nullptr),
               KDN_OK, "forward_keep " + name(d));
        begin_call(wsb);
        expect(kdn_backward_kept(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), lam, S,
                                 fake(20), S, lam, g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7],
                                 W, wsb - 1, nullptr),
               d.B * d.H == 0 ? KDN_OK : KDN_ERR_WORKSPACE, "backward_kept short " + name(d));
    }
}

void varlen_case(int N, int H, int Ttot, int dk, int dv, int C, int var, int qkv) {
    kdn_desc d = desc(N, H, Ttot, dk, dv, C, var, qkv, qkv);
    const size_t ws = kdn_forward_varlen_workspace_bytes(&d);
    begin_call(ws);
    float* lam = static_cast<float*>(fake(7));
    float* S = static_cast<float*>(fake(8));
    expect(kdn_forward_varlen(&d, static_cast<const int32_t*>(fake(30)), Ttot, fake(0), fake(1),
                              fake(2), fake(3), fake(4), fake(5), lam, S, fake(6), S, lam,
                              reinterpret_cast<void*>(kWsBase), ws, nullptr),
           (N == 0 || H == 0) ? KDN_OK : KDN_OK, "varlen " + name(d));
    begin_call(ws);
    if (N > 0 && H > 0)
        expect(kdn_forward_varlen(&d, static_cast<const int32_t*>(fake(30)), Ttot, fake(0),
                                  fake(1), fake(2), fake(3), fake(4), fake(5), lam, S, fake(6), S,
                                  lam, reinterpret_cast<void*>(kWsBase), ws - 1, nullptr),
               KDN_ERR_WORKSPACE, "varlen short " + name(d));
}

}  // namespace

int main() {
    const int dims[] = {32, 64, 128};
    const int chunksz[] = {16, 32, 64};
    const int Ts[] = {0, 1, 63, 64, 65, 1000, 16 * 64 + 37, 4096, 65536};
    for (int dk : dims)
        for (int dv : dims)
            for (int C : chunksz)
                for (int var = 0; var < 2; ++var)
                    for (int qkv = 0; qkv < 2; ++qkv)
                        for (int T : Ts) {
                            kdn_desc d = desc(1, 2, T, dk, dv, C, var, qkv, 1 - qkv);
                            if (kdn_validate(&d) != KDN_OK) continue;
                            forward_case(d);
                        }
    // the benchmark's workloads and a few batch shapes
    forward_case(desc(8, 16, 4096, 128, 128, 64, 0, 1, 1));
    forward_case(desc(8, 16, 4096, 128, 128, 64, 1, 1, 1));
    forward_case(desc(1, 16, 65536, 128, 128, 64, 0, 1, 1));
    forward_case(desc(1, 16, 65536, 128, 128, 64, 1, 1, 1));
    forward_case(desc(0, 4, 100, 64, 64, 64, 0, 0, 0));
    forward_case(desc(3, 0, 100, 64, 64, 64, 0, 0, 0));
    forward_case(desc(2, 4, 2048, 64, 64, 64, 0, 0, 0));
    // invalid descriptors are refused before anything is launched
    const int before = g_launches;
    const kdn_desc bad[] = {desc(1, 1, 10, 48, 64, 64, 0, 0, 0), desc(1, 1, 10, 64, 64, 48, 0, 0, 0),
                            desc(-1, 1, 10, 64, 64, 64, 0, 0, 0), desc(1, 1, -5, 64, 64, 64, 0, 0, 0),
                            desc(1, 1, 10, 64, 64, 64, 2, 0, 0), desc(1, 1, 10, 64, 64, 64, 0, 3, 0),
                            desc(300, 300, 10, 64, 64, 64, 0, 0, 0),
                            desc(1, 1, 10, 128, 128, 64, 0, 0, 0)};
    for (const kdn_desc& d : bad) {
        if (kdn_validate(&d) == KDN_OK) fail("accepted " + name(d));
        if (kdn_forward_workspace_bytes(&d) != 0) fail("workspace for " + name(d));
        if (kdn_forward_segments(&d) != 0) fail("segments for " + name(d));
        expect(kdn_forward(&d, fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), nullptr,
                           nullptr, fake(6), nullptr, nullptr, reinterpret_cast<void*>(kWsBase),
                           size_t(1) << 40, nullptr),
               kdn_validate(&d), "refused " + name(d));
    }
    if (g_launches != before) fail("an invalid descriptor reached a launcher");
    if (kdn_validate(nullptr) != KDN_ERR_NULL) fail("NULL descriptor");
    for (int s = 0; s <= 7; ++s)
        if (!kdn_status_string(static_cast<kdn_status>(s))) fail("status string");
    // packed batches
    for (int C : chunksz)
        for (int var = 0; var < 2; ++var) {
            varlen_case(8, 3, 502, 64, 32, C, var, 1);
            varlen_case(1, 1, 1, 32, 32, C, var, 0);
            varlen_case(5, 2, 0, 128, 128, C, var, 1);
            // one long sequence over few heads: the segmented state pass
            varlen_case(1, 2, 5000, 128, 128, C, var, 1);
            varlen_case(3, 1, 4100, 64, 128, C, var, 0);
        }
    if (g_seg_packed == 0) fail("no packed batch took the segmented state pass");
    std::printf("%d launches checked, %d failures\n", g_launches, g_fail);
    return g_fail == 0 ? 0 : 1;
}
