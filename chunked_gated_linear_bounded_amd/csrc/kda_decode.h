// Single-token step of the recurrence (decode), state in place:
//   S~  = S diag(exp g)                       (decay of every key column)
//   y   = S~ k,   S <- S~ + beta (v - y) k^T  (delta-rule erase and write)
//   o   = S q   = S~ q + beta (v - y) (k . q)
// with S dv x dk in float32 ("Trillion-Parameter MoE Multimodal Models: Engineering
// Long-Context ...", sec. 3.2: a constant-size state per head, updated token by token at
// inference; the gate g = g_min sigmoid(a) of "Trillion-Scale MoE Multimodal Models:
// Practical Techniques ...", sec. 3.2).
//
// The step reads and writes the whole state once, so it is bound by HBM.  One work-group
// per (head, block of 16 value rows); each wave takes 4 rows, its lanes the key channels
// (coalesced 256-byte row segments).  Per row the two dot products y_i = S~_i . k and
// S~_i . q are reduced over the wave together; k . q is reduced once.
#pragma once
#include "kda_device.h"

namespace kda {

// Sum over the 64 lanes of a wave, returned to every lane (wave-uniform).
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror
    x += dpp_mov<0x140>(x);  // row_mirror: every lane holds its row's sum
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return (r0 + r1) + (r2 + r3);
}

template <int DK, int DV, bool F32>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const typename std::conditional<F32, float, __bf16>::type *__restrict__ q,
    const typename std::conditional<F32, float, __bf16>::type *__restrict__ k,
    const typename std::conditional<F32, float, __bf16>::type *__restrict__ v,
    const typename std::conditional<F32, float, __bf16>::type *__restrict__ a,
    const typename std::conditional<F32, float, __bf16>::type *__restrict__ beta,
    float gmin2, int logsig, float *__restrict__ state,
    typename std::conditional<F32, float, __bf16>::type *__restrict__ out)
{
    using E = typename std::conditional<F32, float, __bf16>::type;
    constexpr int CPL = DK / 64;        // key channels per lane
    constexpr int RB = 16;              // value rows per work-group
    constexpr int NB = DV / RB;         // row blocks per head
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t head = blockIdx.x / NB;
    const int r0 = (blockIdx.x % NB) * RB + 4 * wave;  // this wave's 4 rows

    float kc[CPL], qc[CPL], ec[CPL];
    float kq = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        kc[j] = to_f(k[head * DK + c]);
        qc[j] = to_f(q[head * DK + c]);
        ec[j] = ex2(gate_log2(to_f(a[head * DK + c]), gmin2, logsig));  // e^g, in (0, 1]
        kq += kc[j] * qc[j];
    }
    kq = wave_sum(kq);
    const float b = to_f(beta[head]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int i = r0 + rr;
        float *row = state + (head * DV + i) * DK;
        float s[CPL];
        float yk = 0.f, yq = 0.f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            s[j] = row[lane + 64 * j] * ec[j];
            yk += s[j] * kc[j];
            yq += s[j] * qc[j];
        }
        yk = wave_sum(yk);
        yq = wave_sum(yq);
        const float d = b * (to_f(v[head * DV + i]) - yk);
#pragma unroll
        for (int j = 0; j < CPL; ++j) row[lane + 64 * j] = fmaf(d, kc[j], s[j]);
        if (lane == 0) out[head * DV + i] = from_f<E>(fmaf(d, kq, yq));
    }
}

}  // namespace kda
