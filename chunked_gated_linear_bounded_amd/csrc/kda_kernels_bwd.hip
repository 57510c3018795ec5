// Instantiations and launchers of the backward pass (kda_bwd.h).  The recomputation of the
// forward's chunk records and chunk start states runs through the forward's own stages at a
// 16-token chunk (launch_intra, launch_state with `states` set).
#include <hip/hip_runtime.h>

#include "kda_bwd.h"
#include "kda_bwd_chunk.h"
#include "kda_bwd_rev.h"
#include "kda_launch.h"

namespace kda {

template <int DK, int DV, bool F32>
static hipError_t launch_bwd_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const int BH = p.B * p.H, NC = p.T / 16;
    const dim3 rgrid((BH + 7) / 8 * 8 * (DV / 16));  // whole groups of 8 heads (XCD dealing)
    if constexpr (F32)
        hipLaunchKernelGGL((kda_bwd_dstate_kernel<DK, DV, F32>), rgrid, dim3(320), 0, p.stream,
                           reinterpret_cast<const unsigned char *>(p.workspace),
                           reinterpret_cast<const E *>(p.dout), p.dfinal, p.T, BH, p.dstates, p.dinit);
    else
        hipLaunchKernelGGL((kda_bwd_rev_kernel<DK, DV>), rgrid, dim3((DK / 16 + 1) * 64), 0, p.stream,
                           reinterpret_cast<const unsigned char *>(p.workspace),
                           reinterpret_cast<const E *>(p.dout), p.dfinal, p.T, BH, p.dstates, p.dinit);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
static hipError_t by_dims(const LaunchArgs &p) {
    if (p.dk == 64 && p.dv == 64) return launch_bwd_t<64, 64, F32>(p);
    if (p.dk == 64 && p.dv == 128) return launch_bwd_t<64, 128, F32>(p);
    if (p.dk == 128 && p.dv == 64) return launch_bwd_t<128, 64, F32>(p);
    return launch_bwd_t<128, 128, F32>(p);
}

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
    e = launch_state(r);
    if (e != hipSuccess) return e;
    return p.fp32 ? by_dims<true>(p) : by_dims<false>(p);
}

}  // namespace kda
