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
// per (head, block of 16 value rows), 4 rows per wave.  A row of S is read as 16-byte
// pieces, 4 key channels per lane: DK/4 lanes per row, so one wave-wide access covers
// 256/DK rows.  Every load of the wave (its rows of S, and q, k, a, v) is issued before any
// is used, so a wave keeps all its bytes in flight at once; the two dot products of a row,
// y = S~ k and S~ q, are then reduced over the row's lanes, and k . q once.
#pragma once
#include "kda_device.h"

namespace kda {

constexpr int kDecodeRowsPerWave = 4;                       // value rows per wave
constexpr int kDecodeRowsPerBlock = 4 * kDecodeRowsPerWave;  // per 256-thread work-group

// Sum over each group of LPR consecutive lanes (16 or 32), returned to every lane of the group.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);  // row_half_mirror
    x += dpp_mov<0x140>(x);  // row_mirror: every lane holds its 16-lane row's sum
    if constexpr (LPR == 16) {
        return x;
    } else {
        static_assert(LPR == 32, "groups of 16 or 32 lanes");
        const int xi = __builtin_bit_cast(int, x);
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
        return (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
    }
}

// Four consecutive elements as floats (one 8-byte load for bf16, one 16-byte load for fp32).
template <typename E>
__device__ __forceinline__ void load4(const E *__restrict__ p, float (&x)[4]) {
    if constexpr (sizeof(E) == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = v[i];
    } else {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        x[0] = __builtin_bit_cast(float, u.x << 16);
        x[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
        x[2] = __builtin_bit_cast(float, u.y << 16);
        x[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
    }
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
    constexpr int LPR = DK / 4;    // lanes per state row
    constexpr int RPI = 64 / LPR;  // rows per wave-wide access
    constexpr int RPW = kDecodeRowsPerWave;
    constexpr int NI = RPW / RPI;  // accesses per wave
    static_assert(RPW % RPI == 0, "whole accesses per wave");
    constexpr int RB = kDecodeRowsPerBlock;
    constexpr int NB = DV / RB;    // row blocks per head
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __builtin_assume(wave >= 0 && wave < 4);  // 256 threads: the range readfirstlane hides
    const size_t head = blockIdx.x / NB;
    const int c0 = 4 * (lane % LPR);                               // this lane's 4 key channels
    const int rw = (blockIdx.x % NB) * RB + RPW * wave + lane / LPR;  // its row in access 0

    // every load first
    f32x4 st[NI];
    float vr[NI];
#pragma unroll
    for (int x = 0; x < NI; ++x) {
        const int i = rw + RPI * x;
        st[x] = *reinterpret_cast<const f32x4 *>(state + (head * DV + i) * DK + c0);
        vr[x] = to_f(v[head * DV + i]);
    }
    float kc[4], qc[4], ac[4];
    load4(k + head * DK + c0, kc);
    load4(q + head * DK + c0, qc);
    load4(a + head * DK + c0, ac);
    const float b = to_f(beta[head]);

    float ec[4];
    float kq = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ec[j] = ex2(gate_log2(ac[j], gmin2, logsig));  // e^g, in (0, 1]
        kq += kc[j] * qc[j];
    }
    kq = group_sum<LPR>(kq);
#pragma unroll
    for (int x = 0; x < NI; ++x) {
        const int i = rw + RPI * x;
        float s[4];
        float yk = 0.f, yq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[j] = st[x][j] * ec[j];
            yk += s[j] * kc[j];
            yq += s[j] * qc[j];
        }
        yk = group_sum<LPR>(yk);
        yq = group_sum<LPR>(yq);
        const float d = b * (vr[x] - yk);
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = fmaf(d, kc[j], s[j]);
        *reinterpret_cast<f32x4 *>(state + (head * DV + i) * DK + c0) = o;
        if (lane % LPR == 0) out[head * DV + i] = from_f<E>(fmaf(d, kq, yq));
    }
}

}  // namespace kda
