// Chunk-parallel stage: one work-group (4 waves) per (chunk, head, batch).
//
// For one chunk of C tokens (r, s = 0..C-1 local positions, G = inclusive
// log-cumsum of the gate inside the chunk) it computes, all in fp32 with bf16
// (or fp32) MFMA operands:
//   M_rs = sum_c q_rc k_sc e^{G_rc - G_sc}            (s <= r)
//   A_rs = beta_r sum_c k_rc k_sc e^{G_rc - G_sc}     (s <  r)
//   T = (I + A)^-1,  W = T diag(beta) (K e^G),  U~ = T diag(beta) V
//   Q~ = Q e^G,  K^ = K e^{G_last - G},  gamma = e^{G_last}
// and writes them in fragment order to the chunk's workspace record.
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
// UT solve (delta rule in WY form): the 16x16 diagonal blocks of T are solved
// by forward substitution (one lane per column), then the off-diagonal blocks
// level by level, T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, with fp32 MFMAs.
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
    static constexpr int PG = DK + 4;            // sG pitch (floats)
    static constexpr int PQ = DK + (F32 ? 4 : 8);  // q/k pitch (elements)
    static constexpr int PV = DV + (F32 ? 4 : 8);
    static constexpr int PA = C + 4;             // A / T pitch (floats)
    static constexpr int SZ_G = C * PG * 4;
    static constexpr int SZ_TV = C * PA * 4 + C * PV * ES;
    static constexpr int R0 = SZ_G > SZ_TV ? SZ_G : SZ_TV;
    static constexpr int SZ_Q = C * PQ * ES;
    static constexpr int SZ_A = C * PA * 4;
    static constexpr int R1 = SZ_Q > SZ_A ? SZ_Q : SZ_A;
    static constexpr int R2 = C * PQ * ES;
    static constexpr int OFF_R1 = R0, OFF_R2 = R0 + R1, OFF_B = R0 + R1 + R2;
    static constexpr int OFF_SCR = OFF_B + C * 4;
    static constexpr int SMEM = OFF_SCR + 256 * 4;
    static constexpr int VEC = 16 / ES;          // elements per 16-byte access
};

template <int C, int DK, int DV, bool F32>
__global__ __launch_bounds__(256, 2) void kda_intra_kernel(
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ q,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ k,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ v,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ a,
    const typename IntraCfg<C, DK, DV, F32>::E *__restrict__ beta,
    float gmin2, int logsig, int H, int T, unsigned char *__restrict__ ws,
    unsigned long long *__restrict__ counts)
{
    using Cfg = IntraCfg<C, DK, DV, F32>;
    using E = typename Cfg::E;
    using F = Frag<F32>;
    constexpr int NT = Cfg::NT, NDK = Cfg::NDK, NDV = Cfg::NDV, NKB = Cfg::NKB, NTKB = Cfg::NTKB;
    constexpr int PG = Cfg::PG, PQ = Cfg::PQ, PV = Cfg::PV, PA = Cfg::PA, VEC = Cfg::VEC;
    constexpr KdaLayout L = kda_layout(C, DK, DV, Cfg::ES);

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cfg::SMEM];
    float *sG = reinterpret_cast<float *>(smem);                            // R0: G (log2)
    float *sT = reinterpret_cast<float *>(smem);                            // R0: T, after G
    E *sV = reinterpret_cast<E *>(smem + C * PA * 4);                       // R0: V, after G
    E *sQ = reinterpret_cast<E *>(smem + Cfg::OFF_R1);                      // R1: q
    float *sA = reinterpret_cast<float *>(smem + Cfg::OFF_R1);              // R1: A, after q
    E *sK = reinterpret_cast<E *>(smem + Cfg::OFF_R2);                      // R2: k, then beta K~
    float *sB = reinterpret_cast<float *>(smem + Cfg::OFF_B);               // beta
    float *sScr = reinterpret_cast<float *>(smem + Cfg::OFF_SCR);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int n = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int NC = T / C;
    const size_t head = (size_t)b * H + h;
    const size_t tok0 = head * (size_t)T + (size_t)n * C;
    unsigned char *rec = ws + ((size_t)head * NC + n) * L.stride;
    E *wWT = reinterpret_cast<E *>(rec + L.wt);
    E *wQT = reinterpret_cast<E *>(rec + L.qt);
    E *wKH = reinterpret_cast<E *>(rec + L.kh);
    E *wMT = reinterpret_cast<E *>(rec + L.mt);
    float *wGam = reinterpret_cast<float *>(rec + L.gam);
    E *wUT = reinterpret_cast<E *>(rec + L.ut);
    constexpr int TE = 256;  // elements per tile

    // ------------------------------------------------ phase 0: loads, gate, prefix sum
    if (tid < C) sB[tid] = to_f(beta[tok0 + tid]);
    {
        constexpr int LPR = DK / VEC, RPP = 256 / LPR;
        const E *qg = q + tok0 * DK, *kg = k + tok0 * DK;
#pragma unroll
        for (int r0 = 0; r0 < C; r0 += RPP) {
            const int r = r0 + tid / LPR, c = (tid % LPR) * VEC;
            if (r < C) {
                uint4 xq = *reinterpret_cast<const uint4 *>(qg + (size_t)r * DK + c);
                uint4 xk = *reinterpret_cast<const uint4 *>(kg + (size_t)r * DK + c);
                *reinterpret_cast<uint4 *>(sQ + r * PQ + c) = xq;
                *reinterpret_cast<uint4 *>(sK + r * PQ + c) = xk;
            }
        }
    }
    constexpr int VLPR = DV / VEC, VRPP = 256 / VLPR, VN = (C + VRPP - 1) / VRPP;
    uint4 vreg[VN];
    {
        const E *vg = v + tok0 * DV;
#pragma unroll
        for (int it = 0; it < VN; ++it) {
            const int r = it * VRPP + tid / VLPR, c = (tid % VLPR) * VEC;
            if (r < C) vreg[it] = *reinterpret_cast<const uint4 *>(vg + (size_t)r * DV + c);
        }
    }
    gate_cumsum_tile<C, DK, E>(a + tok0 * DK, gmin2, logsig, sG, PG, sScr);  // ends with barrier

    // ------------------------------------------------ phase 1: causal sub-tiles of M and A
    constexpr int MAXJ = (Cfg::NJOB + 3) / 4;
    f32x4 accAs[MAXJ];
    int jobI[MAXJ], jobJ[MAXJ];
    unsigned int nonfinite = 0;
#pragma unroll
    for (int jj = 0; jj < MAXJ; ++jj) {
        const int jb = wave + 4 * jj;
        jobI[jj] = -1;
        if (jb >= Cfg::NJOB) continue;
        int I = 0, rem = jb;
        while (rem > I) { rem -= I + 1; ++I; }
        const int J = rem;
        jobI[jj] = I;
        jobJ[jj] = J;
        const int s = 16 * J + l16, r = 16 * I + l16;
        const float *rho = sG + (16 * I) * PG;
        f32x4 accM = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float cv[8], qv[8], kv[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int c = 32 * kb + 16 * hh + 4 * g;
                float rh[4], gs[4], gr[4], ks[4], kr[4], qr[4];
                ld4(rho + c, rh);
                ld4(sG + s * PG + c, gs);
                ld4(sG + r * PG + c, gr);
                ld4(sK + s * PQ + c, ks);
                ld4(sK + r * PQ + c, kr);
                ld4(sQ + r * PQ + c, qr);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    cv[4 * hh + i] = ks[i] * ex2(rh[i] - gs[i]);   // key, scaled to rho_I
                    const float e = ex2(gr[i] - rh[i]);            // <= 1
                    qv[4 * hh + i] = qr[i] * e;
                    kv[4 * hh + i] = kr[i] * e;
                }
            }
            const F fc = F::make(cv), fq = F::make(qv), fk = F::make(kv);
            if (counts != nullptr && I == J) {
#pragma unroll
                for (int j = 0; j < 8; ++j) nonfinite += !__builtin_isfinite(fc.get(j));
            }
            accM = mma(fc, fq, accM);  // rows s, cols r: M^T
            accA = mma(fk, fc, accA);  // rows r, cols s: A (before beta)
        }
        // M^T tile (st = J, rt = I): keep s <= r
        f32x4 m = accM;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (I == J && (4 * g + i) > l16) m[i] = 0.f;
        st_tile(wMT + (I * (I + 1) / 2 + J) * TE, lane, m);
        // A tile rows r = 16I + 4g + i, cols s = 16J + l16: keep s < r, times beta_r
        f32x4 aa = accA;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool keep = (I > J) || (l16 < 4 * g + i);
            aa[i] = keep ? aa[i] * sB[16 * I + 4 * g + i] : 0.f;
        }
        accAs[jj] = aa;
    }

    // elementwise operands: Q~^T tiles (ct, rt), K^ tiles (st, ct), gamma
    for (int tix = wave; tix < NDK * NT; tix += 4) {
        const int ct = tix / NT, rt = tix % NT;
        const int r = 16 * rt + l16, c = 16 * ct + 4 * g;
        float qr[4], gr[4];
        ld4(sQ + r * PQ + c, qr);
        ld4(sG + r * PG + c, gr);
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = qr[i] * ex2(gr[i]);
        st_tile(wQT + (ct * NT + rt) * TE, lane, o);
    }
    for (int tix = wave; tix < NT * NDK; tix += 4) {
        const int st = tix / NDK, ct = tix % NDK;
        const int c = 16 * ct + l16;
        const float glast = sG[(C - 1) * PG + c];
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int s = 16 * st + 4 * g + i;
            o[i] = to_f(sK[s * PQ + c]) * ex2(glast - sG[s * PG + c]);
        }
        st_tile(wKH + (st * NDK + ct) * TE, lane, o);
    }
    if (tid < DK) wGam[tid] = ex2(sG[(C - 1) * PG + tid]);
    __syncthreads();  // q, raw k and the M/A operands are no longer read

    // ------------------------------------------------ phase 1c: A -> LDS, K -> beta K e^G in place
#pragma unroll
    for (int jj = 0; jj < MAXJ; ++jj) {
        if (jobI[jj] < 0) continue;
        const int I = jobI[jj], J = jobJ[jj];
#pragma unroll
        for (int i = 0; i < 4; ++i) sA[(16 * I + 4 * g + i) * PA + 16 * J + l16] = accAs[jj][i];
    }
    {
        constexpr int LPR = DK / 4, RPP = 256 / LPR;
        for (int r0 = 0; r0 < C; r0 += RPP) {
            const int s = r0 + tid / LPR, c = (tid % LPR) * 4;
            if (s < C) {
                float kr[4], gs[4];
                ld4(sK + s * PQ + c, kr);
                ld4(sG + s * PG + c, gs);
                const float bs = sB[s];
#pragma unroll
                for (int i = 0; i < 4; ++i) sK[s * PQ + c + i] = from_f<E>(bs * kr[i] * ex2(gs[i]));
            }
        }
    }
    __syncthreads();  // G is dead from here on

    // ------------------------------------------------ phase 2: T = (I + A)^-1
    {
        const E *vregE = reinterpret_cast<const E *>(vreg);
        (void)vregE;
#pragma unroll
        for (int it = 0; it < VN; ++it) {
            const int r = it * VRPP + tid / VLPR, c = (tid % VLPR) * VEC;
            if (r < C) *reinterpret_cast<uint4 *>(sV + r * PV + c) = vreg[it];
        }
    }
    // zero the blocks above the diagonal
    for (int x = tid; x < NT * NT * 256; x += 256) {
        const int blk = x >> 8, e = x & 255;
        const int I = blk / NT, J = blk % NT;
        if (I < J) sT[(16 * I + (e >> 4)) * PA + 16 * J + (e & 15)] = 0.f;
    }
    if (wave == 0 && g < NT) {
        // diagonal block I = g, column j = l16, forward substitution
        const int I = g, j = l16;
        const float *Ab = sA + (16 * I) * PA + 16 * I;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc -= Ab[i * PA + kk] * x[kk];
            x[i] = acc;
        }
        float *Tb = sT + (16 * I) * PA + 16 * I;
#pragma unroll
        for (int i = 0; i < 16; ++i) Tb[i * PA + j] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < NT; ++d) {
        const int J = wave, I = wave + d;
        if (I < NT) {
            // X = sum_{K=J}^{I-1} A_IK T_KJ
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
            for (int K = J; K < I; ++K) {
                float av[4];
                ld4(sA + (16 * I + l16) * PA + 16 * K + 4 * g, av);
#pragma unroll
                for (int st = 0; st < 4; ++st)
                    X = mma4(av[st], sT[(16 * K + 4 * g + st) * PA + 16 * J + l16], X);
            }
            // T_IJ = -T_II X
            float tv[4];
            ld4(sT + (16 * I + l16) * PA + 16 * I + 4 * g, tv);
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) Y = mma4(tv[st], X[st], Y);
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[(16 * I + 4 * g + i) * PA + 16 * J + l16] = -Y[i];
        }
        __syncthreads();
    }

    // ------------------------------------------------ phase 3: W^T = (beta K~)^T T^T,  U~ = T (beta V)
    // T fragments: lane l, row r = 16 rt + l16, slots = tokens 32 kb + kslot.
    F tf[NT][NTKB];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int kb = 0; kb < NTKB; ++kb) {
            float x[8];
            const float *row = sT + (16 * rt + l16) * PA + 32 * kb + 4 * g;
            const bool hi = (2 * kb + 1) < NT;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = row[i];
                x[4 + i] = hi ? row[16 + i] : 0.f;
            }
            tf[rt][kb] = F::make(x);
        }
    for (int ct = wave; ct < NDK; ct += 4) {
        F kf[NTKB];
#pragma unroll
        for (int kb = 0; kb < NTKB; ++kb) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = 32 * kb + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
                x[j] = (s < C) ? to_f(sK[s * PQ + 16 * ct + l16]) : 0.f;
            }
            kf[kb] = F::make(x);
        }
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb <= rt / 2; ++kb) acc = mma(kf[kb], tf[rt][kb], acc);
            st_tile(wWT + (ct * NT + rt) * TE, lane, acc);
        }
    }
    for (int vt = wave; vt < NDV; vt += 4) {
        F vf[NTKB];
#pragma unroll
        for (int kb = 0; kb < NTKB; ++kb) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int s = 32 * kb + (j < 4 ? 4 * g + j : 16 + 4 * g + j - 4);
                x[j] = (s < C) ? to_f(sV[s * PV + 16 * vt + l16]) * sB[s] : 0.f;
            }
            vf[kb] = F::make(x);
        }
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb <= rt / 2; ++kb) acc = mma(tf[rt][kb], vf[kb], acc);
            st_tile(wUT + (vt * NT + rt) * TE, lane, acc);
        }
    }
    if (counts != nullptr && nonfinite) atomicAdd(&counts[0], (unsigned long long)nonfinite);
}

}  // namespace kda
