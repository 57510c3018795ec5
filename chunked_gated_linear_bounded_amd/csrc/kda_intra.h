// Chunk-parallel stage: one work-group (8 waves) per (chunk, head, batch).
//
// For one chunk of C tokens (r, s = 0..C-1 local positions, G = inclusive
// log-cumsum of the gate inside the chunk) it computes, fp32 accumulation:
//   M_rs = sum_c q_rc k_sc e^{G_rc - G_sc}            (s <= r)
//   A_rs = beta_r sum_c k_rc k_sc e^{G_rc - G_sc}     (s <  r)
//   T = (I + A)^-1,  Tb = T diag(beta)
//   W = Tb (K e^G),  U~ = Tb V                        (WY form of the delta rule)
//   Oi = M U~        (the chunk's own contribution to its outputs)
//   Qbar = Q e^G - M W,  K^ = K e^{G_last - G},  gamma = e^{G_last}
// so that the sequential stage only has to do, per chunk,
//   U = U~ - W S^T,  O = Oi + Qbar S^T,  S^T <- diag(gamma) S^T + K^^T U.
//
// Gamma scaling without a position-pair path ("Trillion-Scale MoE Multimodal
// Models: Practical Techniques ...", sec. 3.1-3.3; "Breaking Through ...",
// sec. 2.1): the pairwise factor e^{G_r - G_s} is split per channel as
// e^{G_r - rho_I} * e^{rho_I - G_s} with rho_I = G at the first row of r's
// 16-token tile I.  Row factors are <= 1; column factors are <= 1 for earlier
// tiles and at most e^{15 |g_min|} = e^75 on the diagonal tile, inside the bf16
// range because g >= g_min = -5.  So every causal 16x16 sub-tile, diagonal or
// not, is one dense MFMA contraction over the key channels.
//
// Precision: the Gamma-scaled operands of the diagonal sub-tiles of M and A
// (factors up to e^75, outside the fp16 range) enter their products as bf16
// hi + lo pairs (three MFMAs per K-block); M, W and U~ enter M W and M U~ as
// fp16; T diag(beta), K e^G and V are bf16 operands; W, Qbar, K^, U~ and Oi are
// stored as fp16.  Every fp16 operand and stored block is scaled by a power of
// two from its block's largest magnitude, and the scale is undone exactly on the
// fp32 results (here, or in the sequential stage for the stored blocks), so no
// fp16 value depends on the magnitudes of q, k or v.
//
// UT solve: each 16x16 diagonal block of T from the finite product series of
// its strictly lower triangular A block (one wave per block), then the
// off-diagonal blocks level by level, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,
// all with fp32 MFMAs.
#pragma once
#include "kda_device.h"
#include "kda_layout.h"

namespace kda {

template <int C, int DK, int DV, bool F32>
struct IntraCfg {
    using E = typename std::conditional<F32, float, __bf16>::type;
    static constexpr int ES = sizeof(E);
    static constexpr int NT = C / 16, NDK = DK / 16, NDV = DV / 16;
    static constexpr int NKB = DK / 32;          // channel K-blocks
    static constexpr int NTKB = (NT + 1) / 2;    // token K-blocks
    static constexpr int NJOB = NT * (NT + 1) / 2;
    // 64-token chunks: 8 waves, two per SIMD and work-group; with the LDS allowing two work-groups
    // per CU that is four waves per SIMD to hide each other's latencies (with 4-wave work-groups,
    // two per SIMD).  Each row tile is then carried by a pair of waves (HS = 2 halves of the
    // channel K-blocks).  Shorter chunks (one or two row tiles) keep 4 waves: there most waves of
    // an 8-wave group would idle through phases 1 and 2 while still paying their setup.
    static constexpr int NW = NT >= 4 ? 8 : 4, THREADS = NW * 64;
    static constexpr int HS = NW / 4;
    static constexpr int NKBH = NKB / HS;        // channel K-blocks per wave of a row tile
    static constexpr int PG = DK + 4;            // sG pitch (floats)
    static constexpr int PQ = DK + (F32 ? 4 : 8);  // q/k pitch (elements)
    static constexpr int PV = DV + (F32 ? 4 : 8);
    static constexpr int PA = C + 4;             // A / T / M pitch (floats)
    static constexpr int SZ_G = C * PG * 4;
    static constexpr int SZ_TV = C * PA * 4 + C * PV * ES;
    static constexpr int R0 = SZ_G > SZ_TV ? SZ_G : SZ_TV;
    static constexpr int SZ_Q = C * PQ * ES;
    static constexpr int SZ_A = C * PA * 4;
    // phase 1 reuses R1 once q is dead: fp32 key operands K'_J of tiles 0..NT-2 (one 8-value
    // fragment per lane and K-block) and the steps e^{rho_{J+1} - rho_J}
    static constexpr int SZ_X = (NT - 1) * NKB * 512 * 4;
    static constexpr int SZ_XD = SZ_X + (NT - 1) * DK * 4;
    // after the products of phase 1: the second wave of each row tile's pair hands its partial M
    // and A sub-tiles to the first through R1
    static constexpr int SZ_P = HS == 2 ? NJOB * 2 * 256 * 4 : 0;
    // phase 3 with 16-bit operands: M in fp16 (pitch PMH halves) where A was, then the causal
    // (row tile, token K-block) fragments of T diag(beta), each formed once by one wave and read
    // by all (16 bytes per lane)
    static constexpr int PMH = C + 8;
    static constexpr int NTF = NT + (NT - 1) * (NT - 1) / 4;  // sum over rt of rt / 2 + 1
    static constexpr int SZ_TF = F32 ? 0 : NTF * 64 * 16;
    static constexpr int SZ_MT = SZ_A + SZ_TF;
    static constexpr int R1A = SZ_Q > SZ_A ? (SZ_Q > SZ_XD ? SZ_Q : SZ_XD) : (SZ_A > SZ_XD ? SZ_A : SZ_XD);
    static constexpr int R1B = R1A > SZ_P ? R1A : SZ_P;
    static constexpr int R1 = R1B > SZ_MT ? R1B : SZ_MT;
    static constexpr int R2 = C * PQ * ES;
    static constexpr int OFF_R1 = R0, OFF_R2 = R0 + R1, OFF_B = R0 + R1 + R2;

    static constexpr int OFF_TF = OFF_R1 + SZ_A;
    static constexpr int OFF_SCR = OFF_B + C * 4;
    static constexpr int SMEM = OFF_SCR + 256 * 4;
    static constexpr int VEC = 16 / ES;          // elements per 16-byte access
    static constexpr int MAXCT = (NDK + NW - 1) / NW;  // dk tiles per wave
    static constexpr int MAXVT = (NDV + NW - 1) / NW;  // dv slices per wave
};

// Gate pre-activation and its prefix sum from a rank-R factor, on MFMA:
//   a[r][c] = e^{A[c]} sum_j h[r][j] z[c][j],   G[r][c] = sum_{s <= r} gate(a[s][c])  (log2 units)
// (the pre-activation e^A h z of "Trillion-Scale MoE Multimodal Models: Practical Techniques
// ...", sec. 3.2, with h a rank-R factor per token and z the per-head map from it to the key
// channels).  Wave w takes the key-channel tiles w, w + 4, ... for all C rows of the chunk, so it
// reads only its own rows of z, and each channel's whole column is in one wave: the prefix sum
// down the chunk runs in registers (in each lane over its 4 rows, over the 4 lane groups with
// two shuffles, and from tile to tile with the carried total) and G is stored once.  This
// product is private, so its operands use their own K-slot order: slot j of lane group g is
// k = 32 kb + 8 g + j, eight contiguous values, one 16-byte load per fragment straight from
// global memory.  load() only issues the loads (all of them while they fit in 128 registers,
// so the caller can put its own loads behind them); finish() runs the MFMAs, the gate and the
// prefix sum.  R = 16 is half a K-block: lane groups 2 and 3 of the h operand are zero.
template <int C, int DK, typename E, int R>
struct LowRankGate {
    static_assert(R == 16 || R % 32 == 0, "rank 16 or a multiple of 32");
    static constexpr int NT = C / 16, NDK = DK / 16, NCW = (NDK + 3) / 4, NKB = (R + 31) / 32;
    static constexpr bool PRE = NKB * (NT + NCW) * (int)sizeof(Frag<E>) <= 128 * 4;
    static constexpr int NKP = PRE ? NKB : 1;
    Frag<E> fa[NKP][NT], fb[NKP][NCW];
    const E *hp = nullptr, *zp = nullptr;
    int wave = 0;

    __device__ __forceinline__ static Frag<E> ld8(const E *p) {
        if constexpr (std::is_same<E, float>::value) {
            return Frag<float>::load2(p, p + 4);
        } else {
            Frag<E> f;
            f.v = *reinterpret_cast<const typename VecOf<E>::v8 *>(p);
            return f;
        }
    }

    __device__ __forceinline__ void load_kb(int slot, int kb) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) fa[slot][rt] = ld8(hp + (size_t)16 * rt * R + 32 * kb);
#pragma unroll
        for (int ci = 0; ci < NCW; ++ci) {
            const int ct = wave + 4 * ci;
            fb[slot][ci] = ld8(zp + (size_t)16 * (ct < NDK ? ct : 0) * R + 32 * kb);
        }
    }

    // h: the chunk's first row, pitch R; z: [DK][R]
    __device__ __forceinline__ void load(const E *__restrict__ h, const E *__restrict__ z, int w, int lane) {
        const int g = lane >> 4, l16 = lane & 15;
        const int kg = (R == 16 && g >= 2) ? 8 * (g - 2) : 8 * g;  // R = 16: groups 2, 3 reread (then zeroed)
        wave = w;
        hp = h + (size_t)l16 * R + kg;
        zp = z + (size_t)l16 * R + kg;
        if constexpr (PRE) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) load_kb(kb, kb);
        }
    }

    __device__ __forceinline__ void finish(const float *__restrict__ A, float gmin2, int logsig, float *sG, int ldG,
                                           int lane) {
        const int g = lane >> 4, l16 = lane & 15;
        f32x4 acc[NT][NCW];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int ci = 0; ci < NCW; ++ci) acc[rt][ci] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if constexpr (!PRE) load_kb(0, kb);
            const int sl = PRE ? kb : 0;
            if constexpr (R == 16) {
                if (g >= 2) {
#pragma unroll
                    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            if constexpr (std::is_same<E, float>::value) fa[sl][rt].v[j] = 0.f;
                            else fa[sl][rt].v[j] = (E)0.f;
                        }
                }
            }
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int ci = 0; ci < NCW; ++ci) acc[rt][ci] = mma(fa[sl][rt], fb[sl][ci], acc[rt][ci]);
        }
        // one branch on the gate form for the whole scan
        if (logsig) scan<true>(acc, A, gmin2, sG, ldG, lane);
        else scan<false>(acc, A, gmin2, sG, ldG, lane);
    }

    // the gate of each pre-activation and its prefix sum down the chunk, stored as G
    template <bool LS>
    __device__ __forceinline__ void scan(const f32x4 (&acc)[NT][NCW], const float *__restrict__ A, float gmin2,
                                         float *sG, int ldG, int lane) {
        const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
        for (int ci = 0; ci < NCW; ++ci) {
            const int ct = wave + 4 * ci;
            if (ct >= NDK) continue;
            const int c = 16 * ct + l16;
            const float eA = ex2(A[c] * kLog2e);
            float carry = 0.f;  // G of the last row of the tiles above
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = gate_log2_t<LS>(acc[rt][ci][i] * eA, gmin2) + (i ? x[i - 1] : 0.f);
                const float own = x[3];  // inclusive scan of the lane totals over the lane groups
                float t = own;
                const float u1 = __shfl_up(t, 16, 64);
                t += g >= 1 ? u1 : 0.f;
                const float u2 = __shfl_up(t, 32, 64);
                t += g >= 2 ? u2 : 0.f;
                const float add = carry + (t - own);
#pragma unroll
                for (int i = 0; i < 4; ++i) sG[(16 * rt + 4 * g + i) * ldG + c] = x[i] + add;
                carry += __shfl(t, 48 + l16, 64);  // the tile's total, from lane group 3
            }
        }
    }
};

// Fixed-length batches: work-group (x, h, b) takes chunk c0 + x of head (b, h) and writes its
// record at (b H + h) NCw + x, so a launch can cover a window of NCw chunks of every head.
// VL: packed documents (kda_varlen.h).  Work-group x then takes chunk x of the chunk
// table ctab (records at head * NCmax + x); a chunk with fewer than C rows is padded with
// zero q, k, beta and a zero gate, and a table entry with no rows ends the work-group.
// LRK > 0: the gate pre-activation is formed from lrh [B][T][LRK] (shared by the heads), lrz
// [H][DK][LRK] and lrA [H][DK] (LowRankGate) instead of being read from a.
template <int C, int DK, int DV, bool F32, bool VL, int LRK>
__global__ __launch_bounds__((IntraCfg<C, DK, DV, F32>::THREADS), 4) __attribute__((amdgpu_waves_per_eu(4, 4))) void kda_intra_kernel(
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ q,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ k,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ v,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ a,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ beta,
    float gmin2, int logsig, int H, int T, unsigned char *__restrict__ ws,
    unsigned long long *__restrict__ counts, const int4 *__restrict__ ctab, int NCmax, int c0, int NCw,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ lrh,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ lrz, const float *__restrict__ lrA)
{
    constexpr bool LR = LRK > 0;
    static_assert(!(VL && LR), "packed documents take the gate pre-activation as input");
    using Cfg = IntraCfg<C, DK, DV, F32>;
    using E = typename Cfg::E;
    using OW = typename std::conditional<F32, float, __bf16>::type;    // MFMA operands here
    using OH = typename std::conditional<F32, float, _Float16>::type;  // stored Qbar, K^
    using F = Frag<OW>;
    using SP = Split<OW>;
    constexpr int NT = Cfg::NT, NDK = Cfg::NDK, NDV = Cfg::NDV, NKB = Cfg::NKB, NTKB = Cfg::NTKB;
    constexpr int PG = Cfg::PG, PQ = Cfg::PQ, PV = Cfg::PV, PA = Cfg::PA, VEC = Cfg::VEC;
    constexpr int MAXCT = Cfg::MAXCT, MAXVT = Cfg::MAXVT, NW = Cfg::NW, THREADS = Cfg::THREADS, NKBH = Cfg::NKBH;
    constexpr int HS = Cfg::HS;
    static_assert(NKB % HS == 0, "the waves of a row tile take equal shares of the channel K-blocks");
    constexpr KdaLayout L = kda_layout(C, DK, DV, Cfg::ES);
    constexpr int TE = 256;  // elements per tile

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::SMEM];
    float *sG = reinterpret_cast<float *>(smem);                   // R0: G (log2 units)
    float *sT = reinterpret_cast<float *>(smem);                   // R0: T, once G is dead
    E *sV = reinterpret_cast<E *>(smem + C * PA * 4);              // R0: V, once G is dead
    E *sQ = reinterpret_cast<E *>(smem + Cfg::OFF_R1);             // R1: q
    float *sA = reinterpret_cast<float *>(smem + Cfg::OFF_R1);     // R1: A, then M
    float *sXk = reinterpret_cast<float *>(smem + Cfg::OFF_R1);    // R1 in phase 1: shared key operands
    float *sDt = reinterpret_cast<float *>(smem + Cfg::OFF_R1 + Cfg::SZ_X);  // and tile-start steps
    E *sK = reinterpret_cast<E *>(smem + Cfg::OFF_R2);             // R2: k, then K e^G
    float *sB = reinterpret_cast<float *>(smem + Cfg::OFF_B);      // beta
    float *sScr = reinterpret_cast<float *>(smem + Cfg::OFF_SCR);
    float *sP = reinterpret_cast<float *>(smem + Cfg::OFF_R1);     // R1 after phase 1's products: partials
    // block maxima, one per wave: K^ [0, NW), Qbar [NW, 2NW), W [2NW, 3NW), M [3NW, 4NW)
    float *sMaxK = sScr, *sMaxQ = sScr + NW, *sMaxW = sScr + 2 * NW, *sMaxM = sScr + 3 * NW;
    auto max_of = [](const float *m) {
        float x = m[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) x = fmaxf(x, m[w]);
        return x;
    };

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: branches on it stay scalar
    __builtin_assume(wave >= 0 && wave < NW);                   // THREADS threads
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t head = (size_t)b * H + h;
    size_t tok0, recno;
    int nrow = C;  // rows of the chunk that are tokens (compile-time C unless packed)
    if constexpr (VL) {
        const int4 ce = ctab[n];  // same address in every lane: a uniform value
        if (ce.y <= 0) return;    // past the last chunk of the batch
        nrow = ce.y < C ? ce.y : C;
        tok0 = head * (size_t)T + (size_t)ce.x;
        recno = head * (size_t)NCmax + n;
    } else {  // chunk c0 + n of the sequence; the window's records are [head][NCw]
        tok0 = head * (size_t)T + (size_t)(c0 + n) * C;
        recno = head * (size_t)NCw + n;
    }
    unsigned char *rec = ws + recno * L.stride;
    OH *wWT = reinterpret_cast<OH *>(rec + L.wt);
    OH *wQB = reinterpret_cast<OH *>(rec + L.qbt);
    OH *wKH = reinterpret_cast<OH *>(rec + L.kh);
    float *wGam = reinterpret_cast<float *>(rec + L.gam);
    int *wScl = reinterpret_cast<int *>(rec + L.scl);

    // ------------------------------------------------ phase 0: loads, gate, prefix sum
    // Every input load of the chunk (q, k and a as 16-byte accesses, beta) is issued before
    // any of them is consumed, so the chunk pays one memory round trip.  The gate and its
    // prefix sum run in registers and write G once.
    {
        constexpr int LPR = DK / VEC, RPP = THREADS / LPR, NP = (C + RPP - 1) / RPP;
        const E *qg = q + tok0 * DK, *kg = k + tok0 * DK;
        // eight-wave groups with 16-bit inputs run the gate on all their threads, others on 256
        constexpr int GT = (THREADS == 512 && !F32) ? 512 : 256;
        GateScan<C, DK, E, GT> gate;
        LowRankGate<C, DK, E, LR ? LRK : 16> lrt;  // its loads go first: its MFMAs need nothing else
        // the low-rank gate and its prefix sum take the first four waves (256 threads)
        if constexpr (LR) {
            if (wave < 4)
                lrt.load(lrh + ((size_t)b * T + (size_t)(c0 + n) * C) * LRK, lrz + (size_t)h * DK * LRK, wave, lane);
        } else {
            if (GT == THREADS || wave < 4) gate.load(a + tok0 * DK, tid, nrow);
        }
        // loads are unconditional (row indices clamped into the chunk's tokens); only the
        // stores are guarded, and rows past the tokens of a short chunk are stored as zeros
        uint4 xq[NP], xk[NP];
        const E bv = beta[tok0 + (tid < nrow ? tid : nrow - 1)];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = p * RPP + tid / LPR, c = (tid % LPR) * VEC;
            const size_t off = (size_t)(r < nrow ? r : nrow - 1) * DK + c;
            xq[p] = *reinterpret_cast<const uint4 *>(qg + off);
            xk[p] = *reinterpret_cast<const uint4 *>(kg + off);
        }
        // the low-rank gate's MFMAs and prefix sum run while q, k and beta are still in flight
        if constexpr (LR) {
            if (wave < 4) lrt.finish(lrA + (size_t)h * DK, gmin2, logsig, sG, PG, lane);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int r = p * RPP + tid / LPR, c = (tid % LPR) * VEC;
            if (C % RPP == 0 || r < C) {
                uint4 yq = xq[p], yk = xk[p];
                if constexpr (VL) {  // bit masks, not a select of the two arrays (which goes to scratch)
                    const unsigned int mk = r < nrow ? 0xffffffffu : 0u;
                    yq.x &= mk; yq.y &= mk; yq.z &= mk; yq.w &= mk;
                    yk.x &= mk; yk.y &= mk; yk.z &= mk; yk.w &= mk;
                }
                *reinterpret_cast<uint4 *>(sQ + r * PQ + c) = yq;
                *reinterpret_cast<uint4 *>(sK + r * PQ + c) = yk;
            }
        }
        if (tid < C) sB[tid] = (!VL || tid < nrow) ? to_f(bv) : 0.f;
        if constexpr (!LR) {
            if (GT == THREADS || wave < 4) gate.finish(gmin2, logsig, sG, PG, tid, nrow);
        }
        __syncthreads();
    }

    // ------------------------------------------------ phase 1: causal sub-tiles of M and A
    // Wave I owns row tile I and computes M_IJ and A_IJ for every J <= I, every pair referenced
    // to rho_I, the start of the row tile: row operands q e^{G_r - rho_I} and k e^{G_r - rho_I}
    // (<= 1), key operands k_s e^{rho_I - G_s}.  The diagonal tile J = I, whose key factors
    // reach e^{15 |g_min|}, takes bf16 hi + lo operands (three MFMAs); the earlier tiles take
    // single bf16 operands.  Exponentials are paid once per element: wave J's own key operand
    // K'_J = k e^{rho_J - G} goes to LDS in fp32, and a later wave I forms its key operand as
    // K'_J e^{rho_I - rho_J}, the per-channel factor built from the steps between tile starts
    // e^{rho_{J+1} - rho_J}.  Each pair's key operand is still rounded once, from fp32.
    // With eight waves, row tile I is carried by the pair of waves I and 7 - I, each over half
    // the channel K-blocks; the second hands its partial sub-tiles to the first through LDS.
    // Row tile I has I off-diagonal pairs, and waves w and w + 4 share a SIMD, so pairing tile I
    // with tile 3 - I on each SIMD gives every SIMD the same three pairs (pairing waves I and
    // I + 4 put both halves of tile 3 on one SIMD and both of tile 0 on another).
    f32x4 accMs[NT], accAs[NT];  // indexed by J
#pragma unroll
    for (int J = 0; J < NT; ++J) {
        accMs[J] = f32x4{0.f, 0.f, 0.f, 0.f};
        accAs[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    unsigned int nonfinite = 0;
    static_assert(NW == 4 || NT == 4, "eight waves only for four row tiles");
    const int hs = wave >> 2, I = hs ? 3 - (wave & 3) : (wave & 3);  // channel half; row tile
    const int kb0 = hs * NKBH;
    F fqh[NKBH], fkh[NKBH];  // row operands of tile I (single bf16) for the earlier key tiles
    float kown[NKBH][8];     // K'_I in fp32, for the later row tiles
    if (I < NT) {
        const int r = 16 * I + l16;  // this lane's row (A operand) and key (B operand)
        const float *rho = sG + (16 * I) * PG;
#pragma unroll
        for (int kbi = 0; kbi < NKBH; ++kbi) {
            const int kb = kb0 + kbi;
            float qv[8], kv[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = 32 * kb + 16 * hh + 4 * g;
                float rr[4], gr[4], kr[4], qr[4];
                ld4(rho + c, rr);
                ld4(sG + r * PG + c, gr);
                ld4(sK + r * PQ + c, kr);
                ld4(sQ + r * PQ + c, qr);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float e = ex2(gr[i] - rr[i]);  // <= 1
                    qv[4 * hh + i] = qr[i] * e;
                    kv[4 * hh + i] = kr[i] * e;
                    kown[kbi][4 * hh + i] = kr[i] * ex2(rr[i] - gr[i]);  // in [|k|, e^{15 |g_min|} |k|]
                }
            }
            const SP fq = SP::make(qv), fk = SP::make(kv), fc = SP::make(kown[kbi]);
            if (counts != nullptr) {
#pragma unroll
                for (int j = 0; j < 8; ++j) nonfinite += !__builtin_isfinite(fc.hi.get(j));
            }
            fqh[kbi] = fq.hi;
            fkh[kbi] = fk.hi;
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                if (J != I) continue;
                accMs[J] = mma3(fq, fc, accMs[J]);
                accAs[J] = mma3(fk, fc, accAs[J]);
            }
        }
    }
    // steps between tile starts, e^{rho_{J+1} - rho_J} (<= 1, J < NT - 1)
    constexpr int ND = (NT - 1) * DK, NDR = (ND + THREADS - 1) / THREADS;
    float dtab[NDR > 0 ? NDR : 1];
#pragma unroll
    for (int x = 0; x < NDR; ++x) {
        const int e = tid + THREADS * x;
        if (e < ND) {
            const int J = e / DK, c = e % DK;
            dtab[x] = ex2(sG[(16 * J + 16) * PG + c] - sG[(16 * J) * PG + c]);
        }
    }

    // Q e^G as Qbar^T tiles (ct, rt) of this wave's dk tiles, kept in registers until phase 3
    f32x4 qtr[MAXCT][NT];
#pragma unroll
    for (int ci = 0; ci < MAXCT; ++ci) {
        const int ct = wave + NW * ci;
        if (ct >= NDK) continue;
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            const int r = 16 * rt + l16, c = 16 * ct + 4 * g;
            float qr[4], gr[4];
            ld4(sQ + r * PQ + c, qr);
            ld4(sG + r * PG + c, gr);
#pragma unroll
            for (int i = 0; i < 4; ++i) qtr[ci][rt][i] = qr[i] * ex2(gr[i]);
        }
    }
    if constexpr (NT > 1) {
        __syncthreads();  // q is no longer read: its region takes the shared key operands and steps
        if (I < NT - 1) {
#pragma unroll
            for (int kbi = 0; kbi < NKBH; ++kbi) {
                float *xp = sXk + ((I * NKB + kb0 + kbi) * 64 + lane) * 8;
                *reinterpret_cast<f32x4 *>(xp) = f32x4{kown[kbi][0], kown[kbi][1], kown[kbi][2], kown[kbi][3]};
                *reinterpret_cast<f32x4 *>(xp + 4) = f32x4{kown[kbi][4], kown[kbi][5], kown[kbi][6], kown[kbi][7]};
            }
        }
#pragma unroll
        for (int x = 0; x < NDR; ++x) {
            const int e = tid + THREADS * x;
            if (e < ND) sDt[e] = dtab[x];
        }
        __syncthreads();
        if (I < NT) {
#pragma unroll
            for (int kbi = 0; kbi < NKBH; ++kbi) {
                const int kb = kb0 + kbi;
                float f[8];  // e^{rho_I - rho_J} for this lane's channels, J descending
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = 1.f;
#pragma unroll
                for (int J = NT - 2; J >= 0; --J) {
                    if (J >= I) continue;
                    float d0[4], d1[4], x0[4], x1[4];
                    ld4(sDt + J * DK + 32 * kb + 4 * g, d0);
                    ld4(sDt + J * DK + 32 * kb + 16 + 4 * g, d1);
                    const float *xp = sXk + ((J * NKB + kb) * 64 + lane) * 8;
                    ld4(xp, x0);
                    ld4(xp + 4, x1);
                    float cv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        f[j] *= j < 4 ? d0[j] : d1[j - 4];
                        cv[j] = (j < 4 ? x0[j] : x1[j - 4]) * f[j];  // k_s e^{rho_I - G_s} <= |k_s|
                    }
                    const F fc = F::make(cv);
                    accMs[J] = mma(fqh[kbi], fc, accMs[J]);
                    accAs[J] = mma(fkh[kbi], fc, accAs[J]);
                }
            }
        }
    }
    // the pair's partial sub-tiles summed in its first wave: slot I (I + 1) / 2 + J holds M, A
    if constexpr (HS == 2) {
    __syncthreads();  // q and the shared key operands are no longer read: R1 takes the partials
    if (hs == 1 && I < NT) {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            if (J > I) continue;
            float *pp = sP + (size_t)(I * (I + 1) / 2 + J) * 512 + 4 * lane;
            *reinterpret_cast<f32x4 *>(pp) = accMs[J];
            *reinterpret_cast<f32x4 *>(pp + 256) = accAs[J];
        }
    }
    __syncthreads();
    if (hs == 0 && I < NT) {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            if (J > I) continue;
            const float *pp = sP + (size_t)(I * (I + 1) / 2 + J) * 512 + 4 * lane;
            accMs[J] += *reinterpret_cast<const f32x4 *>(pp);
            accAs[J] += *reinterpret_cast<const f32x4 *>(pp + 256);
        }
    }
    }
    float mmax = 0.f;  // largest |M| of row tile I
    if (hs == 0 && I < NT) {
        // element (row r = 16I + 4g + i, col s = 16J + l16): M keeps s <= r, A keeps s < r (times
        // beta_r).  The row tile is made a compile-time value, so only its causal tiles J <= I are
        // touched (with I known only at run time every tile took a select per element).
        auto mask = [&](auto ic) {
            constexpr int IC = decltype(ic)::value;
            if constexpr (IC < NT) {
#pragma unroll
                for (int J = 0; J <= IC; ++J) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 4 * g + i;
                        if (J == IC && l16 > rr) accMs[J][i] = 0.f;
                        accAs[J][i] = (J < IC || l16 < rr) ? accAs[J][i] * sB[16 * IC + rr] : 0.f;
                        mmax = fmaxf(mmax, fabsf(accMs[J][i]));
                    }
                }
            }
        };
        switch (I) {
            case 0: mask(std::integral_constant<int, 0>{}); break;
            case 1: mask(std::integral_constant<int, 1>{}); break;
            case 2: mask(std::integral_constant<int, 2>{}); break;
            default: mask(std::integral_constant<int, 3>{}); break;
        }
    }
    mmax = wave_max(mmax);

    // K^ tiles (st, ct) wait in registers for the chunk's scale; gamma goes to the workspace.
    constexpr int MAXKH = (NT * NDK + NW - 1) / NW;
    f32x4 khr[MAXKH];
    float khmax = 0.f;
#pragma unroll
    for (int xi = 0; xi < MAXKH; ++xi) {
        const int tix = wave + NW * xi;
        if (tix >= NT * NDK) continue;
        const int st = tix / NDK, ct = tix % NDK;
        const int c = 16 * ct + l16;
        const float glast = sG[(C - 1) * PG + c];
        float kv[4];  // k of rows 16 st + 4 g + i, column c
        if constexpr (!F32) {
            const bf16x4 t = ld_tr16<bf16x4>(lds_base(smem) + Cfg::OFF_R2 +
                                             2 * ((16 * st + 4 * g + (l16 >> 2)) * PQ + 16 * ct + 4 * (l16 & 3)));
#pragma unroll
            for (int i = 0; i < 4; ++i) kv[i] = (float)t[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kv[i] = to_f(sK[(16 * st + 4 * g + i) * PQ + c]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * st + 4 * g + i;
            khr[xi][i] = kv[i] * ex2(glast - sG[s * PG + c]);
            khmax = fmaxf(khmax, fabsf(khr[xi][i]));
        }
    }
    khmax = wave_max(khmax);
    if (lane == 0) {
        sMaxK[wave] = khmax;
        sMaxM[wave] = mmax;
    }
    if (tid < DK) wGam[tid] = ex2(sG[(C - 1) * PG + tid]);
    __syncthreads();  // raw k and the shared key operands are no longer read

    // ------------------------------------------------ K^ scaled to fp16 range
    {
        const int sK_ = F32 ? 0 : pow2_scale(max_of(sMaxK));
        if (tid == 0) wScl[2] = sK_;
#pragma unroll
        for (int xi = 0; xi < MAXKH; ++xi) {
            const int tix = wave + NW * xi;
            if (tix >= NT * NDK) continue;
            const int st = tix / NDK, ct = tix % NDK;
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = ldexp2(khr[xi][i], sK_);
            OH *pair = wKH + ((st >> 1) * NDK + ct) * (2 * TE);
            st_half(pair, lane, st & 1, o);
            if (NT & 1) st_half(pair, lane, 1, f32x4{0.f, 0.f, 0.f, 0.f});  // odd tile count: empty partner
        }
    }

    // ------------------------------------------------ phase 1c: A -> LDS, K -> K e^G in place
    if (hs == 0 && I < NT) {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            if (J > I) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) sA[(16 * I + 4 * g + i) * PA + 16 * J + l16] = accAs[J][i];
        }
    }
    {
        constexpr int LPR = DK / 4, RPP = THREADS / LPR;
#pragma unroll
        for (int r0 = 0; r0 < C; r0 += RPP) {
            const int s = r0 + tid / LPR, c = (tid % LPR) * 4;
            if (s < C) {
                float kr[4], gs[4];
                ld4(sK + s * PQ + c, kr);
                ld4(sG + s * PG + c, gs);
#pragma unroll
                for (int i = 0; i < 4; ++i) sK[s * PQ + c + i] = from_f<E>(kr[i] * ex2(gs[i]));
            }
        }
    }
    __syncthreads();  // G is dead from here on

    // ------------------------------------------------ phase 2: T = (I + A)^-1
    {   // V straight into LDS with direct loads (one instruction per 256 bytes of a row);
        // they land while T is being solved and are waited for before phase 3
        constexpr int RB = DV * Cfg::ES, NPR = (RB + 255) / 256;
        const unsigned char *vg = reinterpret_cast<const unsigned char *>(v + tok0 * DV);
        lds_u8 *sVb = lds_base(smem) + C * PA * 4;  // sV, LDS-typed
#pragma unroll
        for (int xi = 0; xi < (C * NPR + NW - 1) / NW; ++xi) {
            const int x = wave + NW * xi;
            if (x >= C * NPR) continue;
            const int r = x / NPR, part = x % NPR, off = part * 256 + lane * 4;
            // rows past a short chunk's tokens repeat its last row (finite; beta = 0 there)
            const int rs = (!VL || r < nrow) ? r : nrow - 1;
            if (off < RB)
                __builtin_amdgcn_global_load_lds(vg + (size_t)rs * RB + off,
                                                 (lds_void *)(sVb + r * PV * Cfg::ES + part * 256), 4, 0, 0);
        }
    }
    if (wave < NT) {
        // Diagonal block I = wave.  N = A_II is strictly lower triangular, so N^16 = 0 and
        // (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) exactly: eight 16x16x16 fp32
        // products.  In the 16x16x4 MFMA layout an accumulator holding Z is Z's B operand
        // and Z^T's A operand as it stands, so Z and Z^T are carried side by side and no
        // product needs a shuffle.  The factors commute, so the running product takes each one
        // as soon as its power exists: four products deep instead of six.
        const int I = wave;
        const float *Ab = sA + (16 * I) * PA + 16 * I;
        f32x4 R, Rt;  // R: N[4g + i][l16]; Rt: N[l16][4g + i]
#pragma unroll
        for (int i = 0; i < 4; ++i) R[i] = Ab[(4 * g + i) * PA + l16];
        {
            float t4[4];
            ld4(Ab + l16 * PA + 4 * g, t4);
#pragma unroll
            for (int i = 0; i < 4; ++i) Rt[i] = t4[i];
        }
        // X Y + Z with X given transposed-accumulator style (xt = D(X^T)) and Y as D(Y)
        auto prod = [](f32x4 xt, f32x4 y, f32x4 z) {
#pragma unroll
            for (int st = 0; st < 4; ++st) z = mma4(xt[st], y[st], z);
            return z;
        };
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 N2 = prod(Rt, R, zero), N2t = prod(R, Rt, zero);
        f32x4 Y, mRt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Y[i] = N2[i] + (4 * g + i == l16 ? 1.f : 0.f);
            mRt[i] = -Rt[i];
        }
        Y = prod(mRt, Y, Y);                                     // (I - N)(I + N^2)
        const f32x4 N4 = prod(N2t, N2, zero), N4t = prod(N2, N2t, zero);
        Y = prod(N4t, Y, Y);                                     // (I + N^4)(...)
        const f32x4 N8t = prod(N4, N4t, zero);                   // (N^8)^T
        Y = prod(N8t, Y, Y);                                     // (I + N^8)(...)
        float *Tb = sT + (16 * I) * PA + 16 * I;
#pragma unroll
        for (int i = 0; i < 4; ++i) Tb[(4 * g + i) * PA + l16] = Y[i];
    }
    barrier_lds();  // V loads stay in flight through the solve
    // X += sum_{K=K0}^{K1-1} A_IK T_KJ and Y += T_IK X (accumulator X as the B operand)
    auto at_sum = [&](int I, int J, int K0, int K1, f32x4 X) {
        for (int K = K0; K < K1; ++K) {
            float av[4];
            ld4(sA + (16 * I + l16) * PA + 16 * K + 4 * g, av);
#pragma unroll
            for (int st = 0; st < 4; ++st) X = mma4(av[st], sT[(16 * K + 4 * g + st) * PA + 16 * J + l16], X);
        }
        return X;
    };
    auto t_times = [&](int I, int K, f32x4 X, f32x4 Y) {
        float tv[4];
        ld4(sT + (16 * I + l16) * PA + 16 * K + 4 * g, tv);
#pragma unroll
        for (int st = 0; st < 4; ++st) Y = mma4(tv[st], X[st], Y);
        return Y;
    };
    auto t_store = [&](int I, int J, f32x4 Y) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(16 * I + 4 * g + i) * PA + 16 * J + l16] = -Y[i];
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (NT == 4) {
        // Two levels, from the 2 x 2 block form of the inverse of a block lower triangular
        // matrix, [[L1, 0], [B, L2]]^-1 = [[T1, 0], [-T2 B T1, T2]], on 32-row halves: first the
        // off-diagonal tiles of T1 and T2 (T_10, T_32), then the four tiles of -T2 (B T1) at
        // once, each wave forming the tiles of B T1 it needs.
        if (wave < 2) {
            const int J = 2 * wave, I = J + 1;
            t_store(I, J, t_times(I, I, at_sum(I, J, J, I, zero4), zero4));
        }
        barrier_lds();
        if (wave < 4) {
            const int I = 2 + (wave >> 1), J = wave & 1;
            const f32x4 X2 = at_sum(2, J, J, 2, zero4);  // (B T1)_{2J}
            f32x4 Y;
            if (I == 2) {
                Y = t_times(2, 2, X2, zero4);
            } else {
                const f32x4 X3 = at_sum(3, J, J, 2, zero4);  // (B T1)_{3J}
                Y = t_times(3, 3, X3, t_times(3, 2, X2, zero4));
            }
            t_store(I, J, Y);
        }
        barrier_lds();
    } else {
#pragma unroll
        for (int d = 1; d < NT; ++d) {
            const int J = wave, I = wave + d;
            if (I < NT) t_store(I, J, t_times(I, I, at_sum(I, J, J, I, zero4), zero4));  // T_IJ = -T_II X
            barrier_lds();
        }
    }
    // A is dead: M takes its place, scaled by 2^sM (the fp16 operand of M W and M U~, whatever the
    // magnitudes of q and k)
    const int sM_ = F32 ? 0 : pow2_scale(max_of(sMaxM));
    OH *sMh = reinterpret_cast<OH *>(smem + Cfg::OFF_R1);  // 16-bit operands: M 2^sM in fp16
    using FV = typename std::conditional<F32, f32x4, bf16x8>::type;  // a bf16 fragment
    FV *sTF = reinterpret_cast<FV *>(smem + Cfg::OFF_TF);
    static_assert(Cfg::NTF <= NW, "one T diag(beta) fragment per wave at most");
    if (hs == 0 && I < NT) {
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            if (J > I) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float m = ldexp2(accMs[J][i], sM_);
                if constexpr (F32) sA[(16 * I + 4 * g + i) * PA + 16 * J + l16] = m;
                else sMh[(16 * I + 4 * g + i) * Cfg::PMH + 16 * J + l16] = (OH)m;
            }
        }
    }
    if constexpr (!F32) {
        // Fragment f of T diag(beta) (the f-th causal (rt, kb) pair, row-major), formed by wave
        // (f + NW / 2) mod NW: the waves that store no M or the fewest tiles of it
        const int f = (wave + NW / 2) % NW;
        int frt = -1, fkb = 0;
        {
            int n = 0;
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb) {
                    if (n == f) { frt = rt; fkb = kb; }
                    ++n;
                }
        }
        if (frt >= 0) {
            float x[8];
            const int r = 16 * frt + l16;
            const bool hi = 2 * fkb + 1 <= frt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s0 = 32 * fkb + 4 * g + i;
                x[i] = sT[r * PA + s0] * sB[s0];
                x[4 + i] = 0.f;
            }
            if (hi) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s1 = 32 * fkb + 16 + 4 * g + i;
                    x[4 + i] = sT[r * PA + s1] * sB[s1];
                }
            }
            sTF[f * 64 + lane] = F::make(x).v;
        }
    }
    wait_vmcnt<0>();  // V has landed in LDS
    __syncthreads();
    const float *sM = sA;

    // ------------------------------------------------ phase 3
    // Fragments indexed by (row tile rt, token K-block kb): lane l holds row r = 16 rt + l16,
    // slots = columns 32 kb + kslot.  tf: T diag(beta); mf: M 2^sM.  The products with M (M W and
    // M U~) take fp16 operands, so one fp16 MFMA (11 significand bits) replaces the two or three
    // bf16 hi + lo products; M, W and U~ each enter scaled by the power of two of their block's
    // maximum, so their fp16 range holds whatever the magnitudes of q, k and v.
    // Only the causal K-blocks kb <= rt / 2 are used.  T and M are stored for blocks on and
    // below the diagonal only; the one block above the diagonal that such a K-block spans
    // (column tile 2 kb + 1 = rt + 1) is zero and is never read.
    using FM = Frag<OH>;  // fp16 (fp32 with fp32 I/O)
    // B operand from column c0 + l16 of a row-major [C][pitch] block of E at byte offset off in
    // LDS: token slots 32 kb + 4 g + j (j < 4) and 32 kb + 16 + 4 g + j - 4, zero past C.  With
    // bf16, two transpose reads of four rows each.
    auto col_frag = [&](int off, int pitch, int kb, int c0) {
        if constexpr (!F32) {
            const lds_u8 *base = lds_base(smem) + off;
            const int r = 32 * kb + 4 * g + (l16 >> 2), c = c0 + 4 * (l16 & 3);
            const bf16x4 lo = ld_tr16<bf16x4>(base + 2 * (r * pitch + c));
            bf16x4 hi = {};
            if (32 * kb + 16 < C) hi = ld_tr16<bf16x4>(base + 2 * ((r + 16) * pitch + c));
            F f;
            f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            return f;
        } else {
            const E *blk = reinterpret_cast<const E *>(smem + off);
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = 32 * kb + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
                x[j] = (s < C) ? to_f(blk[s * pitch + c0 + l16]) : 0.f;
            }
            return F::make(x);
        }
    };
    // Two passes, so that the T and M fragments are never held together: the first forms W^T and
    // W of this wave's dk tile and U~ of its dv slice from T diag(beta), the second the products
    // with M.
    float qbmax = 0.f, wmax = 0.f;
    f32x4 wtr[MAXCT][NT], wrow[MAXCT][NT];  // W^T tiles (ct, rt) and W tiles (rt, ct)
    float wtile[MAXCT];                      // largest |W| of each dk tile
    f32x4 urow[MAXVT][NT];                   // U~ tiles (rt, vt)
    float um[MAXVT];
    {
        F tf[NT][NTKB];
        // fragment (rt, kb): with 16-bit operands read from LDS at its use (the pairs before row
        // tile rt number rt + (rt - 1)^2 / 4)
        auto tfr = [&](int rt, int kb) {
            if constexpr (!F32) {
                F f;
                f.v = sTF[(rt + (rt - 1) * (rt - 1) / 4 + kb) * 64 + lane];
                return f;
            } else {
                return tf[rt][kb];
            }
        };
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                if (kb > rt / 2) continue;
                if constexpr (!F32) {
                    continue;  // read where used
                } else {
                    float x[8];
                    const int r = 16 * rt + l16;
                    const bool hi = 2 * kb + 1 <= rt;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s0 = 32 * kb + 4 * g + i, s1 = s0 + 16;
                        x[i] = sT[r * PA + s0] * sB[s0];
                        x[4 + i] = hi ? sT[r * PA + s1] * sB[s1] : 0.f;
                    }
                    tf[rt][kb] = F::make(x);
                }
            }
#pragma unroll
        for (int ci = 0; ci < MAXCT; ++ci) {
            const int ct = wave + NW * ci;
            wtile[ci] = 0.f;
            if (ct >= NDK) continue;
            F kf[NTKB];  // (K e^G): lane l holds column c = 16 ct + l16 at token slots
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) kf[kb] = col_frag(Cfg::OFF_R2, PQ, kb, 16 * ct);
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                f32x4 accT = {0.f, 0.f, 0.f, 0.f}, accW = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb) {
                    const F t = tfr(rt, kb);
                    accT = mma(kf[kb], t, accT);  // W^T (ct, rt)
                    accW = mma(t, kf[kb], accW);  // W (rt, ct)
                }
                wtr[ci][rt] = accT;
#pragma unroll
                for (int i = 0; i < 4; ++i) wtile[ci] = fmaxf(wtile[ci], fabsf(accT[i]));
                wrow[ci][rt] = accW;
            }
        }
#pragma unroll
        for (int vi = 0; vi < MAXVT; ++vi) {
            const int vt = wave + NW * vi;
            um[vi] = 0.f;
            if (vt >= NDV) continue;
            F vf[NTKB];  // V: lane l holds column 16 vt + l16 at token slots
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) vf[kb] = col_frag(C * PA * 4, PV, kb, 16 * vt);
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb) acc = mma(tfr(rt, kb), vf[kb], acc);
                urow[vi][rt] = acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) um[vi] = fmaxf(um[vi], fabsf(acc[i]));
            }
        }
    }
    {
        FM mf[NT][NTKB];  // M 2^sM
        // fragment (rt, kb): with 16-bit operands two 8-byte reads of the fp16 M at its use
        auto mfr = [&](int rt, int kb) {
            if constexpr (!F32) {
                const OH *p = sMh + (16 * rt + l16) * Cfg::PMH + 32 * kb + 4 * g;
                return 2 * kb + 1 <= rt ? FM::load2(p, p + 16) : FM::load1(p);
            } else {
                return mf[rt][kb];
            }
        };
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                if (kb > rt / 2) continue;
                const int r = 16 * rt + l16;
                const bool hi = 2 * kb + 1 <= rt;
                if constexpr (!F32) {
                    continue;  // read where used
                } else {
                    float y[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s0 = 32 * kb + 4 * g + i, s1 = s0 + 16;
                        y[i] = sM[r * PA + s0];
                        y[4 + i] = hi ? sM[r * PA + s1] : 0.f;
                    }
                    mf[rt][kb] = FM::make(y);
                }
            }
        // dk tiles: Qbar^T = (Q e^G)^T - W^T M^T, kept in registers for the chunk's scale
#pragma unroll
        for (int ci = 0; ci < MAXCT; ++ci) {
            const int ct = wave + NW * ci;
            if (ct >= NDK) continue;
            wmax = fmaxf(wmax, wtile[ci]);
            // W 2^sWa as the A operand of W^T (m = dk, k = token); M W comes out scaled by 2^(sWa + sM)
            const int sWa = F32 ? 0 : pow2_scale(wave_max(wtile[ci]));
            FM wa[NTKB];
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 2 * kb + j / 4;
                    x[j] = (t < NT) ? ldexp2(wrow[ci][t < NT ? t : 0][j % 4], sWa) : 0.f;
                }
                wa[kb] = FM::make(x);
            }
            const int unMW = -(sWa + sM_);
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                f32x4 mw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb) mw = mma(wa[kb], mfr(rt, kb), mw);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    qtr[ci][rt][i] -= ldexp2(mw[i], unMW);
                    qbmax = fmaxf(qbmax, fabsf(qtr[ci][rt][i]));
                }
            }
        }
        // dv slices: U~ and Oi^T = U~^T M^T, scaled per slice to fp16 range
#pragma unroll
        for (int vi = 0; vi < MAXVT; ++vi) {
            const int vt = wave + NW * vi;
            if (vt >= NDV) continue;
            unsigned char *sl = rec + L.region1 + vt * L.slice;
            OH *wU = reinterpret_cast<OH *>(sl + L.ut);
            OH *wO = reinterpret_cast<OH *>(sl + L.oit);
            int *wS = reinterpret_cast<int *>(sl + L.ssc);
            // U~ 2^sU as the A operand of U~^T (m = dv, k = token): the block scale keeps the fp16
            // operand in range whatever the magnitude of v; Oi comes out scaled by 2^sU as well
            const int sU_ = F32 ? 0 : pow2_scale(wave_max(um[vi]));
            FM ua[NTKB];
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 2 * kb + j / 4;
                    x[j] = (t < NT) ? ldexp2(urow[vi][t < NT ? t : 0][j % 4], sU_) : 0.f;
                }
                ua[kb] = FM::make(x);
            }
            f32x4 orow[NT];  // Oi 2^(sU + sM)
            float om = 0.f;
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb) acc = mma(ua[kb], mfr(rt, kb), acc);
                orow[rt] = acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) om = fmaxf(om, fabsf(acc[i]));
            }
            const int sO_ = F32 ? 0 : pow2_scale(wave_max(om));  // Oi is stored scaled by 2^(sU + sM + sO)
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                f32x4 u, o;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    u[i] = ldexp2(urow[vi][rt][i], sU_);
                    o[i] = ldexp2(orow[rt][i], sO_);
                }
                st_tile(wU + rt * TE, lane, u);
                st_tile(wO + rt * TE, lane, o);
            }
            if (lane == 0) {
                wS[0] = sU_;
                wS[1] = sU_ + sM_ + sO_;
                wS[2] = 0;
                wS[3] = 0;
            }
        }
    }
    qbmax = wave_max(qbmax);
    wmax = wave_max(wmax);
    if (lane == 0) {
        sMaxQ[wave] = qbmax;
        sMaxW[wave] = wmax;
    }
    __syncthreads();
    // W^T and Qbar^T scaled to fp16 range, stored as tile pairs along dk
    {
        const int sQ_ = F32 ? 0 : pow2_scale(max_of(sMaxQ));
        const int sW_ = F32 ? 0 : pow2_scale(max_of(sMaxW));
        if (tid == 0) { wScl[0] = sW_; wScl[1] = sQ_; wScl[3] = 0; }
#pragma unroll
        for (int ci = 0; ci < MAXCT; ++ci) {
            const int ct = wave + NW * ci;
            if (ct >= NDK) continue;
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
                f32x4 o, w;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    o[i] = ldexp2(qtr[ci][rt][i], sQ_);
                    w[i] = ldexp2(wtr[ci][rt][i], sW_);
                }
                const int pidx = ((ct >> 1) * NT + rt) * (2 * TE);
                st_half(wQB + pidx, lane, ct & 1, o);
                st_half(wWT + pidx, lane, ct & 1, w);
            }
        }
    }
    if (counts != nullptr && nonfinite) atomicAdd(&counts[0], (unsigned long long)nonfinite);
}

}  // namespace kda
