// Kernel instantiations and launchers for the C ABI in include/kda.h, and the device scratch of
// the allocation-free forward.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_decode.h"
#include "kda_device.h"
#include "kda_intra.h"
#include "kda_launch.h"
#include "kda_state.h"
#include "kda_state_seg.h"
#include "kda_varlen.h"
#include "kda.h"

namespace kda {

// Scratch of kda_chunk_fwd_noalloc: the chunk records of one window of the sequence and, when the
// caller passes no final_state, the state carried from window to window.  Every GPU the library
// runs on holds its own copy for the life of the process.  Host code never uses the array's name
// as an address (on the host it stands for no device memory): noalloc_scratch() hands out the
// device address hipGetSymbolAddress gives for the current device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *dev_ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (dev_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    return hipSuccess;
}

// dst[i] = src[i] (src not NULL) or 0, i < n: the state of an empty sequence, written by a kernel
// rather than a memset or copy node so that it can sit in a captured graph.
__global__ __launch_bounds__(256) void kda_state_fill_kernel(float *__restrict__ dst, const float *__restrict__ src,
                                                            size_t n)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = src != nullptr ? src[i] : 0.f;
}

hipError_t launch_state_fill(float *dst, const float *src, size_t n, hipStream_t stream) {
    if (n == 0 || dst == src) return hipSuccess;
    hipLaunchKernelGGL(kda_state_fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dst, src, n);
    return hipGetLastError();
}

// Standalone gate + per-chunk prefix sum: G_out[t][c] = sum over the chunk of
// g (natural log units).  One work-group per (chunk, head, batch).
template <int C, int DK, bool F32>
__global__ __launch_bounds__(256) void kda_gate_kernel(const typename std::conditional<F32, float, __bf16>::type *__restrict__ a,
                                                      float gmin2, int logsig, int H, int T,
                                                      float *__restrict__ G_out)
{
    constexpr int PG = DK + 4;
    __shared__ __attribute__((aligned(16))) float sG[C * PG];
    const size_t tok0 = ((size_t)blockIdx.z * H + blockIdx.y) * (size_t)T + (size_t)blockIdx.x * C;
    GateScan<C, DK, typename std::conditional<F32, float, __bf16>::type> gate;
    gate.load(a + tok0 * DK, threadIdx.x, C);
    gate.finish(gmin2, logsig, sG, PG, threadIdx.x, C);
    __syncthreads();
    float *o = G_out + tok0 * DK;
    constexpr int LPR = DK / 4, RPP = 256 / LPR;
    for (int r0 = 0; r0 < C; r0 += RPP) {
        const int r = r0 + threadIdx.x / LPR, c = (threadIdx.x % LPR) * 4;
        if (r < C) {
            f32x4 x = *reinterpret_cast<const f32x4 *>(sG + r * PG + c);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] *= kLn2;
            *reinterpret_cast<f32x4 *>(o + (size_t)r * DK + c) = x;
        }
    }
}

template <int C, int DK, bool F32>
static hipError_t launch_gate_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    dim3 grid(p.T / C, p.H, p.B);
    hipLaunchKernelGGL((kda_gate_kernel<C, DK, F32>), grid, dim3(256), 0, p.stream,
                       reinterpret_cast<const E *>(p.a), p.g_min * kLog2e, p.logsig, p.H, p.T, p.G_out);
    return hipGetLastError();
}

// Packed documents (p.cu != NULL): the plan tables sit in the workspace after the records
// (kda_varlen.h): ctab [NCmax] int4, then bnd and coff [N + 1] and seg [P + 1] int; B is 1 and
// T is the length of the packed stream.
struct PlanPtrs {
    int4 *ctab;
    int *bnd, *coff, *seg;
};
static PlanPtrs plan_ptrs(const LaunchArgs &p) {
    unsigned char *base = reinterpret_cast<unsigned char *>(p.workspace) + p.plan_offset;
    int4 *ctab = reinterpret_cast<int4 *>(base);
    int *bnd = reinterpret_cast<int *>(ctab + p.ncmax);
    return PlanPtrs{ctab, bnd, bnd + p.nseq + 1, bnd + 2 * (p.nseq + 1)};
}

template <int C, int DK, int DV, bool F32>
static hipError_t launch_intra_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    if (p.cu != nullptr) {
        const PlanPtrs pl = plan_ptrs(p);
        hipLaunchKernelGGL((kda_varlen_plan_kernel<C>), dim3(1), dim3(1024), 0, p.stream, p.cu, p.nseq, p.T, p.ncmax,
                           pl.bnd, pl.coff);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const int nb = (p.ncmax + 255) / 256;
        hipLaunchKernelGGL((kda_varlen_seg_kernel<C>), dim3(1 + nb + p.nseq), dim3(256), 0, p.stream, pl.bnd, pl.coff,
                           p.nseq, p.nrun, p.ncmax, pl.seg, pl.ctab, nb, p.init_state, p.final_state,
                           p.H * p.dv * p.dk);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((kda_intra_kernel<C, DK, DV, F32, true, 0>), dim3(p.ncmax, p.H, 1),
                           dim3(IntraCfg<C, DK, DV, F32>::THREADS), 0,
                           p.stream, reinterpret_cast<const E *>(p.q), reinterpret_cast<const E *>(p.k),
                           reinterpret_cast<const E *>(p.v), reinterpret_cast<const E *>(p.a),
                           reinterpret_cast<const E *>(p.beta), p.g_min * kLog2e, p.logsig, p.H, p.T,
                           reinterpret_cast<unsigned char *>(p.workspace), p.counts, pl.ctab, p.ncmax, 0, 0,
                           nullptr, nullptr, nullptr);
        return hipGetLastError();
    }
    if (p.lr_h != nullptr) return launch_intra_lowrank(p);
    const int ncw = p.ncw > 0 ? p.ncw : p.T / C;
    dim3 grid(ncw, p.H, p.B);
    hipLaunchKernelGGL((kda_intra_kernel<C, DK, DV, F32, false, 0>), grid, dim3(IntraCfg<C, DK, DV, F32>::THREADS), 0, p.stream,
                       reinterpret_cast<const E *>(p.q), reinterpret_cast<const E *>(p.k),
                       reinterpret_cast<const E *>(p.v), reinterpret_cast<const E *>(p.a),
                       reinterpret_cast<const E *>(p.beta), p.g_min * kLog2e, p.logsig, p.H, p.T,
                       reinterpret_cast<unsigned char *>(p.workspace), p.counts, nullptr, 0, p.c0, ncw, nullptr,
                       nullptr, nullptr);
    return hipGetLastError();
}

// The segmented state stage (kda_state_seg.h) for a whole fixed-length sequence: pass 0 and the
// scan when there are several segments, then pass 1.  The workspace is laid out by kda_fwd_plan.
template <int C, int DK, int DV, bool F32>
static hipError_t launch_state_seg(const LaunchArgs &p, const KdaFwdPlan &plan) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const int U = p.B * p.H, NC = p.T / C;
    unsigned char *ws = reinterpret_cast<unsigned char *>(p.workspace);
    float *segbuf = reinterpret_cast<float *>(ws + plan.seg_off);
    float *phibuf = reinterpret_cast<float *>(ws + plan.phi_off);
    if (plan.nseg > 1) {
        hipLaunchKernelGGL((kda_seg_state_kernel<C, DK, DV, F32, 0>), dim3(U * (plan.nseg - 1)),
                           dim3(SegCfg<C, DK, DV, F32, 0>::THREADS), 0,
                           p.stream, ws, nullptr, nullptr, p.init_state, segbuf, phibuf, U, NC, plan.nseg,
                           plan.seglen, p.T, nullptr);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (plan.nseg > 2) {
            hipLaunchKernelGGL((kda_seg_scan_kernel<DK, DV>), dim3(U * (DV / 16)), dim3(256), 0, p.stream, segbuf,
                               phibuf, plan.nseg);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL((kda_seg_state_kernel<C, DK, DV, F32, 1>), dim3(U * plan.nseg),
                       dim3(SegCfg<C, DK, DV, F32, 1>::THREADS), 0, p.stream, ws,
                       reinterpret_cast<E *>(p.out), p.final_state, p.init_state, segbuf, phibuf, U, NC, plan.nseg,
                       plan.seglen, p.T, p.counts);
    return hipGetLastError();
}

template <int C, int DK, int DV, bool F32>
static hipError_t launch_state_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    const bool vl = p.cu != nullptr;
    if constexpr (kda_seg_supported(kda_layout(C, DK, DV, F32 ? 4 : 2))) {
        // whole fixed-length sequences with outputs: the segmented stage where kda_fwd_plan picks it
        if (!vl && p.states == nullptr && p.ncw == 0 && p.c0 == 0 && p.out != nullptr) {
            const KdaFwdPlan plan = kda_fwd_plan(p.B, p.H, p.T, C, DK, DV, F32 ? 4 : 2);
            if (plan.segmented) return launch_state_seg<C, DK, DV, F32>(p, plan);
        }
    }
    const int BH = vl ? p.nrun * p.H : p.B * p.H;  // units: (run of documents, head) or (batch, head)
    const int groups = (BH + 7) / 8;
    dim3 grid(groups * 8 * (DV / 16));
    const PlanPtrs pl = vl ? plan_ptrs(p) : PlanPtrs{nullptr, nullptr, nullptr, nullptr};
    if (vl)
        hipLaunchKernelGGL((kda_state_kernel<C, DK, DV, F32, true>), grid, dim3(192), 0, p.stream,
                           reinterpret_cast<const unsigned char *>(p.workspace), reinterpret_cast<E *>(p.out),
                           p.final_state, p.init_state, BH, p.T, p.counts, pl.ctab, pl.seg, pl.coff, p.H, p.ncmax,
                           nullptr, 0, 0);
    else
        hipLaunchKernelGGL((kda_state_kernel<C, DK, DV, F32, false>), grid, dim3(192), 0, p.stream,
                           reinterpret_cast<const unsigned char *>(p.workspace), reinterpret_cast<E *>(p.out),
                           p.final_state, p.init_state, BH, p.T, p.counts, nullptr, nullptr, nullptr, p.H, 0,
                           p.states, p.c0, p.ncw > 0 ? p.ncw : p.T / C);
    return hipGetLastError();
}

template <int C, int DK, int DV, bool F32>
static hipError_t launch_stage_t(const LaunchArgs &p, int stage) {
    return stage == 0 ? launch_intra_t<C, DK, DV, F32>(p) : launch_state_t<C, DK, DV, F32>(p);
}

template <int C, bool F32>
static hipError_t dispatch_c(const LaunchArgs &p, int stage) {
    if (p.dk == 64 && p.dv == 64) return launch_stage_t<C, 64, 64, F32>(p, stage);
    if (p.dk == 64 && p.dv == 128) return launch_stage_t<C, 64, 128, F32>(p, stage);
    if (p.dk == 128 && p.dv == 64) return launch_stage_t<C, 128, 64, F32>(p, stage);
    return launch_stage_t<C, 128, 128, F32>(p, stage);
}

template <bool F32>
static hipError_t dispatch_t(const LaunchArgs &p, int stage) {
    if (p.chunk == 16) return dispatch_c<16, F32>(p, stage);
    if (p.chunk == 32) return dispatch_c<32, F32>(p, stage);
    return dispatch_c<64, F32>(p, stage);
}

hipError_t launch_intra(const LaunchArgs &p) { return p.fp32 ? dispatch_t<true>(p, 0) : dispatch_t<false>(p, 0); }
hipError_t launch_state(const LaunchArgs &p) { return p.fp32 ? dispatch_t<true>(p, 1) : dispatch_t<false>(p, 1); }

template <bool F32>
static hipError_t dispatch_gate_t(const LaunchArgs &p) {
    if (p.dk == 64) {
        if (p.chunk == 16) return launch_gate_t<16, 64, F32>(p);
        if (p.chunk == 32) return launch_gate_t<32, 64, F32>(p);
        return launch_gate_t<64, 64, F32>(p);
    }
    if (p.chunk == 16) return launch_gate_t<16, 128, F32>(p);
    if (p.chunk == 32) return launch_gate_t<32, 128, F32>(p);
    return launch_gate_t<64, 128, F32>(p);
}

hipError_t launch_gate_cumsum(const LaunchArgs &p) {
    return p.fp32 ? dispatch_gate_t<true>(p) : dispatch_gate_t<false>(p);
}

template <int DK, int DV, bool F32>
static hipError_t launch_decode_t(const LaunchArgs &p) {
    using E = typename std::conditional<F32, float, __bf16>::type;
    static_assert(DV % kDecodeRowsPerBlock == 0, "whole row blocks");
    const int grid = p.B * p.H * (DV / kDecodeRowsPerBlock);
    hipLaunchKernelGGL((kda_decode_kernel<DK, DV, F32>), dim3(grid), dim3(256), 0, p.stream,
                       reinterpret_cast<const E *>(p.q), reinterpret_cast<const E *>(p.k),
                       reinterpret_cast<const E *>(p.v), reinterpret_cast<const E *>(p.a),
                       reinterpret_cast<const E *>(p.beta), p.g_min * kLog2e, p.logsig, p.state,
                       reinterpret_cast<E *>(p.out));
    return hipGetLastError();
}

template <bool F32>
static hipError_t dispatch_decode_t(const LaunchArgs &p) {
    if (p.dk == 64 && p.dv == 64) return launch_decode_t<64, 64, F32>(p);
    if (p.dk == 64 && p.dv == 128) return launch_decode_t<64, 128, F32>(p);
    if (p.dk == 128 && p.dv == 64) return launch_decode_t<128, 64, F32>(p);
    return launch_decode_t<128, 128, F32>(p);
}

hipError_t launch_decode(const LaunchArgs &p) { return p.fp32 ? dispatch_decode_t<true>(p) : dispatch_decode_t<false>(p); }

}  // namespace kda
