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
//  * Operand types: bf16 (v_mfma_f32_16x16x32_bf16), fp16 (v_mfma_f32_16x16x32_f16),
//    one instruction per K-block; fp32 (eight v_mfma_f32_16x16x4_f32, step j
//    taking slot j).  fp16 operands are always scaled by a power of two chosen
//    from the block's largest magnitude (see pow2_scale), so they cannot
//    overflow; the scale is undone exactly on the fp32 result.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kda {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
// An LDS-typed pointer to a __shared__ object.  Offsets are added to it, never to a generic
// pointer that is cast afterwards: a generic-to-LDS cast carries a null check, and where that
// check does not fold this compiler can emit an instruction with an illegal operand.
template <typename T>
__device__ __forceinline__ lds_u8 *lds_base(T *shared_object) { return (lds_u8 *)shared_object; }

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// gfx950 LDS transpose read of 16-bit values: within each group of 16 lanes, slot k of lane i is
// value i % 4 of the 8 bytes (8-byte aligned) that lane 4 k + i / 4 of the group addresses.  So
// four consecutive rows of one column of a row-major 16-bit block reach lane (g, n) when lane
// (g, s) addresses row r0 + (s >> 2), columns c0 + 4 (s & 3) .. + 3: slot k = X[r0 + k][c0 + n].
// The result is taken as a whole vector of the wanted type: bit-casting its 16-bit elements one
// at a time compiles (with this compiler) to code that converts slot 0 only.
template <typename V>
__device__ __forceinline__ V ld_tr16(const lds_u8 *p) {
    return __builtin_bit_cast(V, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcpf(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float ldexp2(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(_Float16 x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f(float x) { return (E)x; }

// ---------------------------------------------------------------- operand fragments
template <typename T> struct VecOf;
template <> struct VecOf<__bf16> { using v8 = bf16x8; using v4 = bf16x4; };
template <> struct VecOf<_Float16> { using v8 = f16x8; using v4 = f16x4; };

template <typename T> struct Frag {  // 16-bit operand, one 16x16x32 MFMA per K-block
    using V8 = typename VecOf<T>::v8;
    using V4 = typename VecOf<T>::v4;
    V8 v;
    __device__ __forceinline__ static Frag make(const float (&x)[8]) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = (T)x[j];
        return f;
    }
    // slots 0-3 from p0[0..3], slots 4-7 from p1[0..3] (each 8 contiguous bytes)
    __device__ __forceinline__ static Frag load2(const T *p0, const T *p1) {
        V4 a = *reinterpret_cast<const V4 *>(p0);
        V4 b = *reinterpret_cast<const V4 *>(p1);
        Frag f;
        f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
    __device__ __forceinline__ static Frag load1(const T *p0) {  // slots 4-7 zero
        V4 a = *reinterpret_cast<const V4 *>(p0);
        Frag f;
        f.v = __builtin_shufflevector(a, V4{}, 0, 1, 2, 3, 4, 5, 6, 7);
        return f;
    }
    // this lane's fragment from a stored tile pair (8 contiguous values)
    __device__ __forceinline__ static Frag load_pair(const T *pair, int lane) {
        Frag f;
        f.v = *reinterpret_cast<const V8 *>(pair + lane * 8);
        return f;
    }
    __device__ __forceinline__ float get(int j) const { return (float)v[j]; }
    // this lane's 8 values to 8 contiguous elements at base + 8 * lane (one 16-byte store)
    __device__ __forceinline__ void store(T *base, int lane) const {
        *reinterpret_cast<V8 *>(base + lane * 8) = v;
    }
};

template <> struct Frag<float> {  // fp32, eight 16x16x4 MFMAs per K-block
    float v[8];
    __device__ __forceinline__ static Frag make(const float (&x)[8]) {
        Frag f;
#pragma unroll
        for (int j = 0; j < 8; ++j) f.v[j] = x[j];
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
    __device__ __forceinline__ static Frag load_pair(const float *pair, int lane) {
        return load2(pair + lane * 8, pair + lane * 8 + 4);
    }
    __device__ __forceinline__ float get(int j) const { return v[j]; }
    __device__ __forceinline__ void store(float *base, int lane) const {
        *reinterpret_cast<f32x4 *>(base + lane * 8) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(base + lane * 8 + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
};

__device__ __forceinline__ f32x4 mma(const Frag<__bf16> &a, const Frag<__bf16> &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<_Float16> &a, const Frag<_Float16> &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const Frag<float> &a, const Frag<float> &b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
    return c;
}
// Plain fp32 16x16x16 step: lane group g supplies k = 4g + s in step s.
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Split-precision bf16 operands: x = hi + lo, hi = bf16(x), lo = bf16(x - hi),
// good to ~16 significant bits.  A product of two split operands keeps three of
// the four cross terms (the dropped lo*lo is ~2^-16 relative).  With fp32
// operands nothing is split (lo unused).
template <typename T> struct Split {
    Frag<T> hi, lo;
    __device__ __forceinline__ static Split make(const float (&x)[8]) {
        Split s;
        s.hi = Frag<T>::make(x);
        if constexpr (!std::is_same<T, float>::value) {
            float r[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) r[j] = x[j] - s.hi.get(j);
            s.lo = Frag<T>::make(r);
        }
        return s;
    }
};
template <typename T>
__device__ __forceinline__ void st_frag(T *base, int lane, const Frag<T> &f) { f.store(base, lane); }
// This lane's 8 values to LDS at base + 8 * lane elements (one 16-byte store per 8 bytes... of
// 16-bit values, two for float), through an LDS-typed pointer.
__device__ __forceinline__ void st_frag_lds(lds_u8 *base, int lane, const Frag<_Float16> &f) {
    *reinterpret_cast<__attribute__((address_space(3))) f16x8 *>(base + 16 * lane) = f.v;
}
__device__ __forceinline__ void st_frag_lds(lds_u8 *base, int lane, const Frag<float> &f) {
    auto *p = reinterpret_cast<__attribute__((address_space(3))) f32x4 *>(base + 32 * lane);
    p[0] = f32x4{f.v[0], f.v[1], f.v[2], f.v[3]};
    p[1] = f32x4{f.v[4], f.v[5], f.v[6], f.v[7]};
}

template <typename T>
__device__ __forceinline__ f32x4 mma3(const Split<T> &a, const Split<T> &b, f32x4 c) {
    c = mma(a.hi, b.hi, c);
    if constexpr (!std::is_same<T, float>::value) {
        c = mma(a.lo, b.hi, c);
        c = mma(a.hi, b.lo, c);
    }
    return c;
}
template <typename T>
__device__ __forceinline__ f32x4 mma2b(const Frag<T> &a, const Split<T> &b, f32x4 c) {
    c = mma(a, b.hi, c);
    if constexpr (!std::is_same<T, float>::value) c = mma(a, b.lo, c);
    return c;
}

// ---------------------------------------------------------------- reductions and scaling
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// Value of the lane N places lower in the same 16-lane row (0 for the first N lanes of a row).
template <int N>
__device__ __forceinline__ float dpp_row_shr(float x) {
    static_assert(N >= 1 && N <= 15, "row shift");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xF, 0xF, false));
}
// x combined with the DPP-moved copy of itself; lanes whose rows ROWMASK leaves out keep x.
// Unsigned max on the bit patterns: for non-negative floats that are not NaN it orders exactly as
// the float max and needs no NaN quieting.  Lanes the row mask leaves out see 0, the identity of
// the unsigned max, so the move folds into one v_max_u32_dpp.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ unsigned dpp_max_with(unsigned x) {
    const unsigned y = (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWMASK, 0xF, false);
    return x > y ? x : y;
}
// Maximum over the 64 lanes of a wave of x >= 0 (not NaN; +inf allowed), returned to every lane
// (wave-uniform): four steps inside each 16-lane row, then the gfx9 row broadcasts carry row 0
// into row 1 and row 2 into row 3 (lane 15, resp. 47) and row 1 into rows 2 and 3 (lane 31), so
// lane 63 holds the maximum; one readlane instead of four.  Every caller passes a maximum of
// magnitudes taken with fmaxf, which never returns NaN unless all its inputs are NaN.
__device__ __forceinline__ float wave_max(float xf) {
    unsigned x = __builtin_bit_cast(unsigned, xf);
    x = dpp_max_with<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
    x = dpp_max_with<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
    x = dpp_max_with<0x141, 0xF>(x);  // row_half_mirror
    x = dpp_max_with<0x140, 0xF>(x);  // row_mirror: every lane has its row's max
    x = dpp_max_with<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x = dpp_max_with<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane((int)x, 63));
}
// Power-of-two exponent s that maps magnitudes <= m into [2^13, 2^14) at the
// top: x * 2^s is exact and stays below the fp16 maximum (65504).
__device__ __forceinline__ int pow2_scale(float m) { return 14 - __builtin_amdgcn_frexp_expf(m); }

// Whether the wave-wide maximum of x (x >= 0, not NaN) lies in [lo, hi): no lane at or above hi,
// some lane at or above lo.  Two compares and two lane masks; no data crosses lanes.
__device__ __forceinline__ bool wave_max_in(float x, float lo, float hi) {
    return __builtin_amdgcn_ballot_w64(x >= hi) == 0 && __builtin_amdgcn_ballot_w64(x >= lo) != 0;
}

// Store / load this lane's 4 values of a fragment-ordered 16x16 tile.
template <typename T>
__device__ __forceinline__ void st_tile(T *tile, int lane, f32x4 x) {
    if constexpr (std::is_same<T, float>::value) {
        *reinterpret_cast<f32x4 *>(tile + lane * 4) = x;
    } else {
        typename VecOf<T>::v4 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = (T)x[i];
        *reinterpret_cast<typename VecOf<T>::v4 *>(tile + lane * 4) = b;
    }
}
// Store this lane's 4 values of tile `half` (0: tile 2p, 1: tile 2p+1) of a tile pair.
template <typename T>
__device__ __forceinline__ void st_half(T *pair, int lane, int half, f32x4 x) {
    st_tile(pair + lane * 4 + half * 4, lane, x);  // lands at pair + 8 lane + 4 half
}
__device__ __forceinline__ f32x4 ld_tile(const float *tile, int lane) {
    return *reinterpret_cast<const f32x4 *>(tile + lane * 4);
}
template <typename T>
__device__ __forceinline__ f32x4 ld_tile(const T *tile, int lane) {
    const typename VecOf<T>::v4 b = *reinterpret_cast<const typename VecOf<T>::v4 *>(tile + lane * 4);
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)b[i];
    return x;
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

// ---------------------------------------------------------------- direct global->LDS loads

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt unconstrained): all but the N most recent
// vector-memory instructions of this wave have completed.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Work-group barrier that orders LDS traffic only.  __syncthreads() is a fenced
// barrier: every wave first drains all of its vector-memory operations, which
// would also retire direct global->LDS loads that are meant to stay in flight
// across the barrier.  Here each wave waits for its own LDS reads and writes
// (lgkmcnt(0)) and the compiler keeps memory accesses on their side of the
// barrier; a wave that filled LDS with direct loads must wait for them itself
// (wait_vmcnt) before arriving.  Global stores are not made visible by it.
__device__ __forceinline__ void barrier_lds() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt 63 and expcnt 7 leave the rest alone
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------- the gate
// g in log2 units (g * log2 e).  Bounded: g_min * sigmoid(a).  Log-sigmoid:
// log sigmoid(a) = -(max(-a, 0) + log(1 + e^-|a|)), never overflows.
template <bool LOGSIG>
__device__ __forceinline__ float gate_log2_t(float a, float gmin2) {
    float g;
    if constexpr (!LOGSIG) g = gmin2 * rcpf(1.f + ex2(-a * kLog2e));
    else g = -(fmaxf(-a, 0.f) * kLog2e + lg2(1.f + ex2(-fabsf(a) * kLog2e)));
    // rounded here: a prefix sum adds it as a value and never fuses its product into an fma, so
    // every caller (with or without a guard on the row) sums the same values
    asm volatile("" : "+v"(g));
    return g;
}
__device__ __forceinline__ float gate_log2(float a, float gmin2, int logsig) {
    return logsig ? gate_log2_t<true>(a, gmin2) : gate_log2_t<false>(a, gmin2);
}

// Gate and inclusive prefix sum over the C rows of one chunk, per channel, held in registers:
// G[r][c] = sum_{s <= r} g2[s][c] (log2 units).  NTH threads (256, or 512 with 16-bit inputs);
// the 16 lanes of each row group rg = tid / 16 take one group of VEC channels (rg + NTH / 16 p
// in pass p) and lane m = tid % 16 takes the RPL = C / 16 consecutive rows m RPL ...  Each lane
// loads its values with 16-byte loads (8-byte ones with 512 threads, so that all of them share
// the work), sums its own rows, and the lane totals are prefix-summed across the row group with
// four DPP row shifts.  load() only issues the loads, so a caller can put other loads in flight
// before finish() consumes them.
template <int C, int DK, typename E, int NTH = 256>
struct GateScan {
    static_assert(NTH == 256 || (NTH == 512 && sizeof(E) == 2), "256 threads, or 512 with 16-bit inputs");
    static constexpr int LB = NTH == 512 ? 8 : 16;    // bytes per load
    static constexpr int VEC = LB / (int)sizeof(E);   // channels per load
    static constexpr int NG = DK / VEC;               // channel groups
    static constexpr int NRG = NTH / 16;              // row groups
    static constexpr int NPASS = (NG + NRG - 1) / NRG;
    static constexpr int RPL = C / 16;
    using LT = typename std::conditional<LB == 16, uint4, uint2>::type;               // rows per lane
    static_assert(C % 16 == 0 && DK % VEC == 0 && VEC % 4 == 0, "chunk and channel tiling");
    LT raw[NPASS][RPL];

    // a: this chunk's [C][DK] block, of which the first nrow rows are tokens (the others are
    // never read: their loads repeat the last token row)
    __device__ __forceinline__ void load(const E *__restrict__ a, int tid, int nrow) {
        const int rg = tid >> 4, m = tid & 15;
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int gi = rg + NRG * p, gc = gi < NG ? gi : NG - 1;  // clamped: loads stay in bounds
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const int r = m * RPL + j;
                raw[p][j] = *reinterpret_cast<const LT *>(a + (size_t)(r < nrow ? r : nrow - 1) * DK + gc * VEC);
            }
        }
    }

    // G over the chunk; rows from nrow on get g = 0, so G stays flat past the last token.  One
    // branch on the gate form for the whole scan (a per-element choice compiles to a branch pair
    // per element).
    __device__ __forceinline__ void finish(float gmin2, int logsig, float *sG, int ldG, int tid, int nrow) {
        if (logsig) finish_t<true>(gmin2, sG, ldG, tid, nrow);
        else finish_t<false>(gmin2, sG, ldG, tid, nrow);
    }
    template <bool LS>
    __device__ __forceinline__ void finish_t(float gmin2, float *sG, int ldG, int tid, int nrow) {
        const int rg = tid >> 4, m = tid & 15;
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int gi = rg + NRG * p;
            if (gi >= NG) continue;  // uniform over the 16 lanes of a row group
            float gv[RPL][VEC];
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const E *e = reinterpret_cast<const E *>(&raw[p][j]);
#pragma unroll
                for (int c = 0; c < VEC; ++c)
                    gv[j][c] = (m * RPL + j < nrow ? gate_log2_t<LS>(to_f(e[c]), gmin2) : 0.f) + (j ? gv[j - 1][c] : 0.f);
            }
            scan_store(gv, sG, ldG, gi, m);
        }
    }

    // gv holds this lane's rows already summed within the lane; add the totals of the lanes
    // before it in the row group (inclusive DPP scan) and store G.
    __device__ __forceinline__ static void scan_store(float (&gv)[RPL][VEC], float *sG, int ldG, int gi, int m) {
#pragma unroll
        for (int c = 0; c < VEC; ++c) {
            const float own = gv[RPL - 1][c];
            float t = own;  // inclusive prefix of the lane totals over m
            t += dpp_row_shr<1>(t);
            t += dpp_row_shr<2>(t);
            t += dpp_row_shr<4>(t);
            t += dpp_row_shr<8>(t);
            const float before = t - own;
#pragma unroll
            for (int j = 0; j < RPL; ++j) gv[j][c] += before;
        }
#pragma unroll
        for (int j = 0; j < RPL; ++j) {
            float *dst = sG + (m * RPL + j) * ldG + gi * VEC;
#pragma unroll
            for (int c = 0; c < VEC; c += 4)
                *reinterpret_cast<f32x4 *>(dst + c) = f32x4{gv[j][c], gv[j][c + 1], gv[j][c + 2], gv[j][c + 3]};
        }
    }
};

}  // namespace kda
