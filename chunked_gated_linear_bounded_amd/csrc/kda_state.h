// Sequential stage: inter-chunk state propagation fused with the output combine.
//
// The state S^T (dk x dv, fp32) of one head is split into dv/16 independent
// column slices (column j of S^T only ever depends on column j of U and of
// S^T itself).  One work-group per (head, slice) walks the chunks in order:
//   U   = U~ - W S^T                              (C x 16)
//   O^T = Oi^T + (S^T)^T Qbar^T                   (16 x C)  -> out
//   S^T = diag(gamma) S^T + K^^T U                (dk x 16)
// with W, Qbar, K^, gamma, U~ and Oi = M U~ from the chunk-parallel stage
// ("Trillion-Parameter MoE Multimodal Models: Engineering Long-Context ...",
// sec. 3.2: a constant-size state updated chunk by chunk).
//
// The slice of S^T stays in the compute wave's registers for the whole
// sequence in accumulator layout; by the slot convention of kda_device.h the
// same registers (rounded to the operand type) are the B operand of W S^T and
// the A operand of (S^T)^T Qbar^T, and U's accumulators are the B operand of
// K^^T U -- no shuffles, no LDS round trips.  U enters K^^T U as a bf16
// hi + lo pair.
//
// Work-group = 2 waves: wave 0 computes, wave 1 copies the next chunk's record
// into the other half of a double buffer in LDS; one barrier per chunk hands
// the buffers over.  Work-group ids are mapped so that all slices of a head
// land on one XCD and share its L2.
#pragma once
#include "kda_device.h"
#include "kda_layout.h"

namespace kda {

template <int C, int DK, int DV, bool F32>
struct StateCfg {
    using E = typename std::conditional<F32, float, __bf16>::type;
    static constexpr int ES = sizeof(E);
    static constexpr KdaLayout L = kda_layout(C, DK, DV, ES);
    static constexpr int BUF = (int)(L.region1 + L.slice);
    static constexpr int LDS_MAX = 160 * 1024;
    static constexpr int NBUF = (2 * BUF <= LDS_MAX) ? 2 : 1;
    static constexpr int SMEM = NBUF * BUF;
    static constexpr int NS = DV / 16;
};

// Copy BYTES (a multiple of 16) from global memory to LDS with one wave, in
// batches of 16-byte loads that are all issued before the first store.
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(unsigned char *dst, const unsigned char *__restrict__ src, int lane) {
    static_assert(BYTES % 16 == 0, "16-byte units");
    constexpr int UNITS = BYTES / 16, PER = (UNITS + 63) / 64, B = 16;
#pragma unroll
    for (int b0 = 0; b0 < PER; b0 += B) {
        uint4 x[B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int u = (b0 + i) * 64 + lane;
            if (b0 + i < PER && u < UNITS) x[i] = *reinterpret_cast<const uint4 *>(src + (size_t)u * 16);
        }
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int u = (b0 + i) * 64 + lane;
            if (b0 + i < PER && u < UNITS) *reinterpret_cast<uint4 *>(dst + u * 16) = x[i];
        }
    }
}

// One chunk's record for one value slice: region 1, then the slice.
template <int R1, int SL>
__device__ __forceinline__ void load_record(unsigned char *dst, const unsigned char *__restrict__ rec,
                                            size_t slice_off, int lane) {
    copy_to_lds<R1>(dst, rec, lane);
    copy_to_lds<SL>(dst + R1, rec + slice_off, lane);
}

template <int C, int DK, int DV, bool F32>
__global__ __launch_bounds__(128, 1) void kda_state_kernel(
    const unsigned char *__restrict__ ws, typename StateCfg<C, DK, DV, F32>::E *__restrict__ out,
    float *__restrict__ final_state, int BH, int T, unsigned long long *__restrict__ counts)
{
    using Cfg = StateCfg<C, DK, DV, F32>;
    using E = typename Cfg::E;
    using F = Frag<F32>;
    using SP = Split<F32>;
    constexpr KdaLayout L = Cfg::L;
    constexpr int NT = C / 16, NDK = DK / 16, NKB = DK / 32, NTKB = (NT + 1) / 2;
    constexpr int NS = Cfg::NS, BUF = Cfg::BUF, NBUF = Cfg::NBUF;
    constexpr int TE = 256;
    constexpr int R1B = (int)L.region1, SLB = (int)L.slice;

    // all slices of a head on one XCD: work-group ids are dealt round-robin to the 8 XCDs
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int hb = (local / NS) * 8 + xcd, slice = local % NS;
    if (hb >= BH) return;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::SMEM];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int NC = T / C;
    const unsigned char *rec0 = ws + (size_t)hb * NC * L.stride;
    const size_t soff = L.region1 + (size_t)slice * L.slice;
    const int j0 = 16 * slice;

    if (wave == 1 && NC > 0) load_record<R1B, SLB>(smem, rec0, soff, lane);
    __syncthreads();

    f32x4 S[NDK];
#pragma unroll
    for (int mt = 0; mt < NDK; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    unsigned int nonfinite = 0;

    for (int n = 0; n < NC; ++n) {
        const unsigned char *cur = smem + (NBUF == 2 ? (n & 1) * BUF : 0);
        if (wave == 1) {
            if (NBUF == 2 && n + 1 < NC) {
                const unsigned char *rec = rec0 + (size_t)(n + 1) * L.stride;
                load_record<R1B, SLB>(smem + ((n + 1) & 1) * BUF, rec, soff, lane);
            }
        } else {
            const E *bWT = reinterpret_cast<const E *>(cur + L.wt);
            const E *bQB = reinterpret_cast<const E *>(cur + L.qbt);
            const E *bKH = reinterpret_cast<const E *>(cur + L.kh);
            const float *bG = reinterpret_cast<const float *>(cur + L.gam);
            const float *bU = reinterpret_cast<const float *>(cur + L.region1 + L.ut);
            const float *bO = reinterpret_cast<const float *>(cur + L.region1 + L.oit);
            const int lo = lane * 4;

            // state slice as operand (B of W S^T, A of (S^T)^T Qbar^T)
            F Sb[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = S[2 * kb + j / 4][j % 4];
                Sb[kb] = F::make(x);
            }
            // U = U~ - W S^T   (tiles over tokens)
            f32x4 U[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    acc = mma(F::load2(bWT + ((2 * kb) * NT + tt) * TE + lo,
                                       bWT + ((2 * kb + 1) * NT + tt) * TE + lo), Sb[kb], acc);
                const f32x4 ut = ld_tile(bU + tt * TE, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) U[tt][i] = ut[i] - acc[i];
            }
            SP Ub[NTKB];
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 2 * kb + j / 4;
                    x[j] = (t < NT) ? U[t < NT ? t : 0][j % 4] : 0.f;
                }
                Ub[kb] = SP::make(x);
            }
            // O^T = Oi^T + (S^T)^T Qbar^T, one 16 x 16 tile per 16 tokens
            const size_t trow = (size_t)hb * T + (size_t)n * C;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 acc = ld_tile(bO + tt * TE, lane);
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    acc = mma(Sb[kb], F::load2(bQB + ((2 * kb) * NT + tt) * TE + lo,
                                               bQB + ((2 * kb + 1) * NT + tt) * TE + lo), acc);
                // lane holds out[token 16 tt + l16][value j0 + 4g + i]
                E *op = out + (trow + 16 * tt + l16) * DV + j0 + 4 * g;
                if constexpr (F32) {
                    *reinterpret_cast<f32x4 *>(op) = acc;
                    if (counts != nullptr) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) nonfinite += !__builtin_isfinite(acc[i]);
                    }
                } else {
                    bf16x4 bo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) bo[i] = (__bf16)acc[i];
                    *reinterpret_cast<bf16x4 *>(op) = bo;
                    if (counts != nullptr) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) nonfinite += !__builtin_isfinite((float)bo[i]);
                    }
                }
            }
            // S^T = diag(gamma) S^T + K^^T U
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) {
                const f32x4 gm = *reinterpret_cast<const f32x4 *>(bG + 16 * mt + 4 * g);
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = S[mt][i] * gm[i];
#pragma unroll
                for (int kb = 0; kb < NTKB; ++kb) {
                    const E *p0 = bKH + ((2 * kb) * NDK + mt) * TE + lo;
                    const F kf = (2 * kb + 1 < NT) ? F::load2(p0, bKH + ((2 * kb + 1) * NDK + mt) * TE + lo)
                                                   : F::load1(p0);
                    acc = mma2b(kf, Ub[kb], acc);
                }
                S[mt] = acc;
            }
        }
        __syncthreads();
        if (NBUF == 1) {
            if (wave == 1 && n + 1 < NC) {
                const unsigned char *rec = rec0 + (size_t)(n + 1) * L.stride;
                load_record<R1B, SLB>(smem, rec, soff, lane);
            }
            __syncthreads();
        }
    }
    if (wave == 0) {
        if (final_state != nullptr) {
            // final_state[hb][value j0 + l16][key 16 mt + 4g + i] = S^T[key][value]
            float *fp = final_state + ((size_t)hb * DV + j0 + l16) * DK + 4 * g;
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) *reinterpret_cast<f32x4 *>(fp + 16 * mt) = S[mt];
        }
        if (counts != nullptr && nonfinite) atomicAdd(&counts[1], (unsigned long long)nonfinite);
    }
}

}  // namespace kda
