// Instantiations and launcher of the chunk-parallel stage with the gate pre-activation formed
// from a rank-R factor (R in {16, 32, 64, 128}); its own translation unit so the two build in
// parallel.
#include <hip/hip_runtime.h>

#include "kda_intra.h"
#include "kda_launch.h"

namespace kda {

template <int C, int DK, int DV, bool F32, int R>
static hipError_t launch_lr_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const int ncw = p.ncw > 0 ? p.ncw : p.T / C;
    hipLaunchKernelGGL((kda_intra_kernel<C, DK, DV, F32, false, R>), dim3(ncw, p.H, p.B),
                       dim3(IntraCfg<C, DK, DV, F32>::THREADS), 0,
                       p.stream, reinterpret_cast<const E *>(p.q), reinterpret_cast<const E *>(p.k),
                       reinterpret_cast<const E *>(p.v), nullptr, reinterpret_cast<const E *>(p.beta),
                       p.g_min * kLog2e, p.logsig, p.H, p.T, reinterpret_cast<unsigned char *>(p.workspace), p.counts,
                       nullptr, 0, p.c0, ncw, reinterpret_cast<const E *>(p.lr_h), reinterpret_cast<const E *>(p.lr_z),
                       p.lr_A);
    return hipGetLastError();
}

template <int C, int DK, int DV, bool F32>
static hipError_t by_rank(const LaunchArgs &p) {
    switch (p.rank) {
    case 16: return launch_lr_t<C, DK, DV, F32, 16>(p);
    case 32: return launch_lr_t<C, DK, DV, F32, 32>(p);
    case 64: return launch_lr_t<C, DK, DV, F32, 64>(p);
    default: return launch_lr_t<C, DK, DV, F32, 128>(p);
    }
}

template <int C, bool F32>
static hipError_t by_dims(const LaunchArgs &p) {
    if (p.dk == 64 && p.dv == 64) return by_rank<C, 64, 64, F32>(p);
    if (p.dk == 64 && p.dv == 128) return by_rank<C, 64, 128, F32>(p);
    if (p.dk == 128 && p.dv == 64) return by_rank<C, 128, 64, F32>(p);
    return by_rank<C, 128, 128, F32>(p);
}

template <bool F32>
static hipError_t by_chunk(const LaunchArgs &p) {
    if (p.chunk == 16) return by_dims<16, F32>(p);
    if (p.chunk == 32) return by_dims<32, F32>(p);
    return by_dims<64, F32>(p);
}

hipError_t launch_intra_lowrank(const LaunchArgs &p) { return p.fp32 ? by_chunk<true>(p) : by_chunk<false>(p); }

}  // namespace kda
