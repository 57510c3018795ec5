// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// MFMA conventions used throughout (one wave = 64 lanes, l = lane, g = l / 16):
//  * 16x16 accumulator ("D") tile: lane l holds rows 4g+i (i = 0..3) of column l%16.
//  * A K-block of 32: lane l supplies 8 operand values ("slots" j = 0..7) for row
//    (A operand) or column (B operand) l%16.  Slot j of lane group g stands for
//    k index  kslot(g, j) = (j < 4 ? 4g + j : 16 + 4g + (j - 4)).
//    The hardware pairs A and B values of the same lane group and slot, so any
//    bijection works as long as both operands use it; this one makes the slots
//    of lane l equal to its accumulator rows in tiles 2kb and 2kb+1.  Hence
//    an accumulator tile pair of X can be fed back, with no data movement, as
//    the B operand of X (k = row of X) or the A operand of X^T (m = column of X).
//  * bf16 operands use v_mfma_f32_16x16x32_bf16 (one instruction per K-block);
//    fp32 operands use eight v_mfma_f32_16x16x4_f32, step j taking slot j.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcpf(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// ---------------------------------------------------------------- operand fragments
template <bool F32> struct Frag;

template <> struct Frag<false> {  // bf16, one 16x16x32 MFMA per K-block
    bf16x8 v;
    __device__ __forceinline__ static Frag make(const float (&x)[8]) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = (__bf16)x[j];
        return f;
    }
    __device__ __forceinline__ static Frag zero() { Frag f; f.v = bf16x8{}; return f; }
    // slots 0-3 from p0[0..3], slots 4-7 from p1[0..3] (each 8 contiguous bytes)
    __device__ __forceinline__ static Frag load2(const __bf16 *p0, const __bf16 *p1) {
        bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
        bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
        Frag f;
        f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
    __device__ __forceinline__ static Frag load1(const __bf16 *p0) {  // slots 4-7 zero
        bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
        Frag f;
        f.v = __builtin_shufflevector(a, bf16x4{}, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
    __device__ __forceinline__ float get(int j) const { return (float)v[j]; }
};

template <> struct Frag<true> {  // fp32, eight 16x16x4 MFMAs per K-block
    float v[8];
    __device__ __forceinline__ static Frag make(const float (&x)[8]) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = x[j];
        return f;
    }
    __device__ __forceinline__ static Frag zero() {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = 0.f;
        return f;
    }
    __device__ __forceinline__ static Frag load2(const float *p0, const float *p1) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p0);
        f32x4 b = *reinterpret_cast<const f32x4 *>(p1);
        Frag f;
#pragma unroll
        for (int j = 0; j < 4; ++j) { f.v[j] = a[j]; f.v[4 + j] = b[j]; }
        return f;
    }
    __device__ __forceinline__ static Frag load1(const float *p0) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p0);
        Frag f;
#pragma unroll
        for (int j = 0; j < 4; ++j) { f.v[j] = a[j]; f.v[4 + j] = 0.f; }
        return f;
    }
    __device__ __forceinline__ float get(int j) const { return v[j]; }
};

__device__ __forceinline__ f32x4 mma(const Frag<false> &a, const Frag<false> &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<true> &a, const Frag<true> &b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}
// Split-precision operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi),
// good to about 16 significant bits.  A product of two split operands keeps
// three of the four cross terms (hi*hi + lo*hi + hi*lo); the dropped lo*lo is
// ~2^-16 relative.  With fp32 operands no split is needed (lo unused).
template <bool F32> struct Split {
    Frag<F32> hi, lo;
    __device__ __forceinline__ static Split make(const float (&x)[8]) {
        Split s;
        s.hi = Frag<F32>::make(x);
        if constexpr (!F32) {
            float r[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) r[j] = x[j] - s.hi.get(j);
            s.lo = Frag<F32>::make(r);
        }
        return s;
    }
};
template <bool F32>
__device__ __forceinline__ f32x4 mma3(const Split<F32> &a, const Split<F32> &b, f32x4 c) {
    c = mma(a.hi, b.hi, c);
    if constexpr (!F32) {
        c = mma(a.lo, b.hi, c);
        c = mma(a.hi, b.lo, c);
    }
    return c;
}
// one split operand (the other exact in the operand type): hi*b + lo*b
template <bool F32>
__device__ __forceinline__ f32x4 mma2a(const Split<F32> &a, const Frag<F32> &b, f32x4 c) {
    c = mma(a.hi, b, c);
    if constexpr (!F32) c = mma(a.lo, b, c);
    return c;
}
template <bool F32>
__device__ __forceinline__ f32x4 mma2b(const Frag<F32> &a, const Split<F32> &b, f32x4 c) {
    c = mma(a, b.hi, c);
    if constexpr (!F32) c = mma(a, b.lo, c);
    return c;
}

// Plain fp32 16x16x16 step: lane group g supplies k = 4g + s in step s.
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Store / load this lane's 4 values of a fragment-ordered 16x16 tile.
__device__ __forceinline__ void st_tile(__bf16 *tile, int lane, f32x4 x) {
    bf16x4 b;
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = (__bf16)x[i];
    *reinterpret_cast<bf16x4 *>(tile + lane * 4) = b;
}
__device__ __forceinline__ void st_tile(float *tile, int lane, f32x4 x) {
    *reinterpret_cast<f32x4 *>(tile + lane * 4) = x;
}
__device__ __forceinline__ f32x4 ld_tile(const __bf16 *tile, int lane) {
    bf16x4 b = *reinterpret_cast<const bf16x4 *>(tile + lane * 4);
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)b[i];
    return x;
}
__device__ __forceinline__ f32x4 ld_tile(const float *tile, int lane) {
    return *reinterpret_cast<const f32x4 *>(tile + lane * 4);
}

// Four consecutive elements as floats (8 or 16 contiguous bytes).
__device__ __forceinline__ void ld4(const __bf16 *p, float (&x)[4]) {
    bf16x4 b = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)b[i];
}
__device__ __forceinline__ void ld4(const float *p, float (&x)[4]) {
    f32x4 b = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = b[i];
}

// ---------------------------------------------------------------- the gate
// g in log2 units (g * log2 e).  Bounded: g_min * sigmoid(a).  Log-sigmoid:
// log sigmoid(a) = -(max(-a, 0) + log(1 + e^-|a|)), never overflows.
__device__ __forceinline__ float gate_log2(float a, float gmin2, int logsig) {
    if (!logsig) return gmin2 * rcpf(1.f + ex2(-a * kLog2e));
    return -(fmaxf(-a, 0.f) * kLog2e + lg2(1.f + ex2(-fabsf(a) * kLog2e)));
}

// Gate and inclusive prefix sum over the C rows of one chunk, per channel:
// sG[r * ldG + c] = sum_{s <= r} g2[s][c] (log2 units).  Threads: 256; thread t
// takes channel t % DK and the t / DK-th segment of rows; segment totals are
// combined through sScratch (>= 256 floats).  Ends with a barrier.
template <int C, int DK, typename E>
__device__ __forceinline__ void gate_cumsum_tile(const E *__restrict__ a, float gmin2, int logsig,
                                                 float *sG, int ldG, float *sScratch) {
    static_assert(256 % DK == 0, "DK must divide 256");
    constexpr int NSEG = 256 / DK;
    static_assert(C % NSEG == 0, "chunk too small for the scan split");
    constexpr int RPS = C / NSEG;
    const int tid = threadIdx.x;
    const int c = tid % DK, seg = tid / DK;
    const int r0 = seg * RPS;
    float av[RPS];
#pragma unroll
    for (int r = 0; r < RPS; ++r) av[r] = to_f(a[(size_t)(r0 + r) * DK + c]);
    float run = 0.f;
#pragma unroll
    for (int r = 0; r < RPS; ++r) {
        run += gate_log2(av[r], gmin2, logsig);
        sG[(r0 + r) * ldG + c] = run;
    }
    sScratch[seg * DK + c] = run;
    __syncthreads();
    float off = 0.f;
    for (int s = 0; s < seg; ++s) off += sScratch[s * DK + c];
    if (seg > 0) {
#pragma unroll
        for (int r = 0; r < RPS; ++r) sG[(r0 + r) * ldG + c] += off;
    }
    __syncthreads();
}

}  // namespace kda
