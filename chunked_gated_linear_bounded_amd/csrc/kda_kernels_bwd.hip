// Instantiations and launchers of the backward pass (kda_bwd.h, kda_bwd_rev.h, kda_bwd_chunk.h).
// The recomputation of the forward's chunk records and chunk start states runs through the
// forward's own stages at a 16-token chunk (launch_intra, launch_state with `states` set).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_bwd.h"
#include "kda_bwd_chunk.h"
#include "kda_bwd_rev.h"
#include "kda_launch.h"

namespace kda {

// The reverse pass (state gradients) on stream st.
template <int DK, int DV, bool F32>
static hipError_t launch_rev_t(const LaunchArgs &p, hipStream_t st) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const int BH = p.B * p.H;
    const dim3 rgrid((BH + 7) / 8 * 8 * (DV / 16));  // whole groups of 8 heads (XCD dealing)
    if constexpr (F32)
        hipLaunchKernelGGL((kda_bwd_dstate_kernel<DK, DV, F32>), rgrid, dim3(320), 0, st,
                           reinterpret_cast<const unsigned char *>(p.workspace),
                           reinterpret_cast<const E *>(p.dout), p.dfinal, p.T, BH, p.dstates, p.dinit);
    else
        hipLaunchKernelGGL((kda_bwd_rev_kernel<DK, DV>), rgrid, dim3((DK / 16 + 1) * 64), 0, st,
                           reinterpret_cast<const unsigned char *>(p.workspace),
                           reinterpret_cast<const E *>(p.dout), p.dfinal, p.T, BH, p.dstates, p.dinit);
    return hipGetLastError();
}

// The chunk-parallel gradient stage on p.stream.
template <int DK, int DV, bool F32>
static hipError_t launch_chunk_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const int BH = p.B * p.H, NC = p.T / 16;
    if constexpr (F32)  // fp32 inputs: every product in fp32 (their 1e-4 bar)
        hipLaunchKernelGGL((kda_bwd_chunk_kernel<DK, DV, F32>), dim3(NC, BH), dim3(512), 0, p.stream,
                           reinterpret_cast<const E *>(p.q), reinterpret_cast<const E *>(p.k),
                           reinterpret_cast<const E *>(p.v), reinterpret_cast<const E *>(p.a),
                           reinterpret_cast<const E *>(p.beta), reinterpret_cast<const E *>(p.dout), p.g_min * kLog2e,
                           p.g_min, p.logsig, p.T, p.states, p.dstates, p.dq, p.dk_, p.dv_, p.da, p.dbeta);
    else  // bf16 inputs: state operands in registers, shared operands split once in LDS
        hipLaunchKernelGGL((kda_bwd_chunk16_kernel<DK, DV>), dim3(NC, BH), dim3(256), 0, p.stream,
                           reinterpret_cast<const E *>(p.q), reinterpret_cast<const E *>(p.k),
                           reinterpret_cast<const E *>(p.v), reinterpret_cast<const E *>(p.a),
                           reinterpret_cast<const E *>(p.beta), reinterpret_cast<const E *>(p.dout), p.g_min * kLog2e,
                           p.g_min, p.logsig, p.T, p.states, p.dstates, p.dq, p.dk_, p.dv_, p.da, p.dbeta);
    return hipGetLastError();
}

template <bool F32>
static hipError_t rev_by_dims(const LaunchArgs &p, hipStream_t st) {
    if (p.dk == 64 && p.dv == 64) return launch_rev_t<64, 64, F32>(p, st);
    if (p.dk == 64 && p.dv == 128) return launch_rev_t<64, 128, F32>(p, st);
    if (p.dk == 128 && p.dv == 64) return launch_rev_t<128, 64, F32>(p, st);
    return launch_rev_t<128, 128, F32>(p, st);
}

template <bool F32>
static hipError_t chunk_by_dims(const LaunchArgs &p) {
    if (p.dk == 64 && p.dv == 64) return launch_chunk_t<64, 64, F32>(p);
    if (p.dk == 64 && p.dv == 128) return launch_chunk_t<64, 128, F32>(p);
    if (p.dk == 128 && p.dv == 64) return launch_chunk_t<128, 64, F32>(p);
    return launch_chunk_t<128, 128, F32>(p);
}

// A second stream per device (default priority, not synchronising with the null stream) for the
// reverse pass, and the two events that fork it off the caller's stream and join it back.  Made
// on a device's first backward call and kept until the process ends.  The mutex keeps each call's
// record-then-wait pairs together when several host threads share a device.
namespace {
struct SideStream {
    hipStream_t st = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::mutex m;
    bool ok = false;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::once_flag g_side_once[kMaxDevices];

SideStream *side_stream() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    SideStream *ss = &g_side[dev];
    std::call_once(g_side_once[dev], [ss]() {
        ss->ok = hipStreamCreateWithFlags(&ss->st, hipStreamNonBlocking) == hipSuccess &&
                 hipEventCreateWithFlags(&ss->fork, hipEventDisableTiming) == hipSuccess &&
                 hipEventCreateWithFlags(&ss->join, hipEventDisableTiming) == hipSuccess;
    });
    return ss->ok ? ss : nullptr;
}
}  // namespace

// p.workspace holds the 16-token chunk records; p.states / p.dstates the chunk states.
hipError_t launch_bwd(const LaunchArgs &p) {
    LaunchArgs r = p;  // recompute: chunk records, then the chunk start states (no outputs)
    r.chunk = 16;
    r.out = nullptr;
    r.final_state = nullptr;
    r.counts = nullptr;
    r.cu = nullptr;
    r.lr_h = nullptr;
    hipError_t e = launch_intra(r);
    if (e != hipSuccess) return e;
    // The state recompute and the reverse pass read only the chunk records and write disjoint
    // parts of the workspace, so they run side by side: the reverse pass on the second stream.
    // Both are serial chains that leave most of a compute unit idle, and a work-group of each fits
    // on one compute unit.  Without a second stream they run one after the other.
    SideStream *ss = side_stream();
    if (ss == nullptr) {
        e = launch_state(r);
        if (e != hipSuccess) return e;
        e = p.fp32 ? rev_by_dims<true>(p, p.stream) : rev_by_dims<false>(p, p.stream);
        if (e != hipSuccess) return e;
        return p.fp32 ? chunk_by_dims<true>(p) : chunk_by_dims<false>(p);
    }
    std::lock_guard<std::mutex> lock(ss->m);
    if ((e = hipEventRecord(ss->fork, p.stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->st, ss->fork, 0)) != hipSuccess) return e;
    e = p.fp32 ? rev_by_dims<true>(p, ss->st) : rev_by_dims<false>(p, ss->st);
    if (e != hipSuccess) return e;
    e = launch_state(r);
    if (e != hipSuccess) return e;
    if ((e = hipEventRecord(ss->join, ss->st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(p.stream, ss->join, 0)) != hipSuccess) return e;
    return p.fp32 ? chunk_by_dims<true>(p) : chunk_by_dims<false>(p);
}

}  // namespace kda
