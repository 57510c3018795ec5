// Chunk-parallel stage of the backward pass for bf16 inputs: the gradients of one 16-token chunk
// of one head from the state the chunk starts from and the gradient of the state it ends in
// (the math is the one written out at the top of kda_bwd.h; "Breaking Through Trillion-Parameter
// Multimodal MoE ...", sec. 2.1: the training scripts above the operator need exactly these
// gradients).
//
// Data movement is laid out for the MI355X rather than for the arithmetic's order:
//   - four waves per work-group and under 80 KB of LDS, so two work-groups share a CU and one
//     computes while the other waits for its 148 KB of state, state gradient and inputs;
//   - each wave reads the state blocks it multiplies straight from global memory into registers,
//     in the MFMA operand order: the rows of its 16-wide value tiles for the key-deep products
//     (U, K^ dS') and the columns of its 16-wide key tiles for the value-deep ones (dQ~, dW, dK^);
//     each block is split once into bf16 hi + lo (about 16 significand bits, the full fp32 range);
//   - every operand that all waves share (K e^{G-G0}, K e^{G0-G}, Q e^{G-G0}, K e^G, K^, W, U, dU,
//     dW) is formed once, split once and kept in LDS as hi and lo rows, which an MFMA operand reads
//     as one 16-byte row piece per lane;
//   - the 16-deep products of the pairwise terms (dM, dP against the scaled q and k) run on
//     16x16x16 bf16 MFMAs with both fp32 operands split into hi + lo (three MFMAs; one fp32
//     16x16x4 MFMA takes four times the cycles of a bf16 16x16x16 one for a quarter of the depth).
//     The others (the solve, W, U~, M^T dO, dX, dY, dA) stay on fp32 16x16x4 MFMAs: dv = diag(b)
//     T^T dU is small beside the terms of dU, and T = (I + A)^-1 and M can hold entries far above 1,
//     so a 16-bit operand anywhere in dU or a product with T costs dv, dk, da and dbeta their
//     precision.  Either way an accumulator tile is a B operand as it stands (lane group g holds
//     rows 4 g .. 4 g + 3 of its column, the B layout of both MFMAs);
//   - T = (I + A)^-1 is the exact finite series (I - N)(I + N^2)(I + N^4)(I + N^8), N = A strictly
//     lower, on one wave while the others form dQ~.
#pragma once
#include "kda_bwd.h"

namespace kda {

struct HL8 {  // one 32-deep block of an MFMA operand, split: x = hi + lo
    bf16x8 h, l;
};

// Two values per packed conversion: hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ HL8 split8(const float (&x)[8]) {
    HL8 s;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const f32x2 v = {x[2 * p], x[2 * p + 1]};
        const bf16x2 hp = __builtin_convertvector(v, bf16x2);
        const bf16x2 lp = __builtin_convertvector(v - __builtin_convertvector(hp, f32x2), bf16x2);
        s.h[2 * p] = hp[0];
        s.h[2 * p + 1] = hp[1];
        s.l[2 * p] = lp[0];
        s.l[2 * p + 1] = lp[1];
    }
    return s;
}

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 8 values of row r, columns c .. c + 7, into an LDS block of hi rows followed by lo rows.
template <int L>
__device__ __forceinline__ void st_hl8(__bf16 *buf, int r, int c, const float (&x)[8]) {
    const HL8 s = split8(x);
    *reinterpret_cast<bf16x8 *>(buf + r * L + c) = s.h;
    *reinterpret_cast<bf16x8 *>(buf + 16 * L + r * L + c) = s.l;
}

// An accumulator tile (lane (g, n) holds rows 4 g + i of column n) into columns c0 .. c0 + 15.
template <int L>
__device__ __forceinline__ void st_acc_hl(__bf16 *buf, f32x4 acc, int c0, int lane) {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 h = (__bf16)acc[i];
        buf[(4 * g + i) * L + c0 + n] = h;
        buf[16 * L + (4 * g + i) * L + c0 + n] = (__bf16)(acc[i] - (float)h);
    }
}

// acc += A B over K = 32 NB.  A: rows of an LDS hi/lo block (output row m = lane & 15 reads its
// row); B: register fragments, block b of lane (g, n) holding B[32 b + 8 g + s][n].
template <int NB, int L>
__device__ __forceinline__ f32x4 mm_hl_reg(f32x4 acc, const __bf16 *A, const HL8 (&B)[NB], int lane) {
    const __bf16 *ah = A + (lane & 15) * L + 8 * (lane >> 4);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const bf16x8 x = ld8(ah + 32 * b), y = ld8(ah + 16 * L + 32 * b);
        acc = mfma32(x, B[b].h, acc);
        acc = mfma32(y, B[b].h, acc);
        acc = mfma32(x, B[b].l, acc);
    }
    return acc;
}
// The same with A exact in bf16 (an input row block, no lo part).
template <int NB, int L>
__device__ __forceinline__ f32x4 mm_h_reg(f32x4 acc, const __bf16 *A, const HL8 (&B)[NB], int lane) {
    const __bf16 *ah = A + (lane & 15) * L + 8 * (lane >> 4);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const bf16x8 x = ld8(ah + 32 * b);
        acc = mfma32(x, B[b].h, acc);
        acc = mfma32(x, B[b].l, acc);
    }
    return acc;
}
// acc += A Bs^T over K = 32 NB with both operands rows of LDS blocks: A[m][k] = A_rows[m][k],
// B[k][n] = Bs[n][k].  HA / HB: the operand has a lo part (else it is exact in bf16).
template <int NB, int LA, int LB, bool HA, bool HB>
__device__ __forceinline__ f32x4 mm_rows(f32x4 acc, const __bf16 *A, const __bf16 *Bs, int lane) {
    const __bf16 *ap = A + (lane & 15) * LA + 8 * (lane >> 4);
    const __bf16 *bp = Bs + (lane & 15) * LB + 8 * (lane >> 4);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const bf16x8 ah = ld8(ap + 32 * b), bh = ld8(bp + 32 * b);
        acc = mfma32(ah, bh, acc);
        if constexpr (HA) acc = mfma32(ld8(ap + 16 * LA + 32 * b), bh, acc);
        if constexpr (HB) acc = mfma32(ah, ld8(bp + 16 * LB + 32 * b), acc);
    }
    return acc;
}

// acc += A B over 16 with fp32 16x16x4 MFMAs: step i takes k = 4 g + i from lane group g.
// a(i) = A[lane & 15][4 g + i], b(i) = B[4 g + i][lane & 15].
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const FA &a, const FB &b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(i), b(i), acc, 0, 0, 0);
    return acc;
}

// The same operands for a 16x16x16 bf16 MFMA (f(i), i = 0..3: this lane's k = 4 g + i), split.
struct HL4 {
    bf16x4 h, l;
};
template <typename F>
__device__ __forceinline__ HL4 split_at(const F &f) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = f(i);
    HL4 s;
    split4(x, s.h, s.l);
    return s;
}
// acc += A B over 16, both operands split (lo x lo dropped).
__device__ __forceinline__ f32x4 mm16_hl(f32x4 acc, const HL4 &a, const HL4 &b) {
    acc = mfma16(a.h, b.h, acc);
    acc = mfma16(a.l, b.h, acc);
    return mfma16(a.h, b.l, acc);
}

// Row block of the stored state [DV][DK] for value rows j0 .. j0 + 15 (B operand of a key-deep
// product, k = key): block b of lane (g, n) = S[j0 + n][32 b + 8 g .. + 7], 32-byte loads.
template <int DK>
__device__ __forceinline__ void load_rows(const float *S, int j0, int lane, float (&x)[DK / 32][8]) {
    const float *p = S + (size_t)(j0 + (lane & 15)) * DK + 8 * (lane >> 4);
#pragma unroll
    for (int b = 0; b < DK / 32; ++b) {
        const f32x4 u = *reinterpret_cast<const f32x4 *>(p + 32 * b);
        const f32x4 w = *reinterpret_cast<const f32x4 *>(p + 32 * b + 4);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            x[b][s] = u[s];
            x[b][4 + s] = w[s];
        }
    }
}
// Column block for key columns c0 .. c0 + 15 (B operand of a value-deep product, k = value):
// block b of lane (g, n) = S[32 b + 8 g + s][c0 + n]; 16 lanes read 64 contiguous bytes of a row.
template <int DK, int DV>
__device__ __forceinline__ void load_cols(const float *S, int c0, int lane, float (&x)[DV / 32][8]) {
    const float *p = S + (size_t)(8 * (lane >> 4)) * DK + c0 + (lane & 15);
#pragma unroll
    for (int b = 0; b < DV / 32; ++b)
#pragma unroll
        for (int s = 0; s < 8; ++s) x[b][s] = p[(size_t)(32 * b + s) * DK];
}

template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void kda_bwd_chunk16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const __bf16 *__restrict__ a, const __bf16 *__restrict__ beta, const __bf16 *__restrict__ dout, float gmin2,
    float gmin, int logsig, int T, const float *__restrict__ states, const float *__restrict__ dstates,
    float *__restrict__ dq, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ da,
    float *__restrict__ dbeta)
{
    constexpr int C = 16, NW = 4, NTH = 64 * NW;
    constexpr int NDK = DK / 16, NDV = DV / 16, TK = NDK / NW, TV = NDV / NW;  // tiles per wave
    constexpr int NBK = DK / 32, NBV = DV / 32;                                 // 32-deep blocks
    constexpr int DM = DK > DV ? DK : DV;
    constexpr int LK = DK + 8, LV = DV + 8, LM = DM + 8, LG = DK + 4, P16 = 17;
    static_assert(NDK % NW == 0 && NDV % NW == 0, "head dimensions of 64 or 128");
    constexpr int UK = C * DK / 8, UV = C * DV / 8;  // 16-byte input units
    static_assert(UK <= NTH && UV <= NTH, "one input unit per thread");

    __shared__ __attribute__((aligned(16))) float sG[C * LG];  // a, then G (log2 units), then dG
    __shared__ __attribute__((aligned(16))) __bf16 sQ[C * LK], sK[C * LK], sA[C * LK], sV[C * LV], sO[C * LV];
    __shared__ __attribute__((aligned(16))) __bf16 bA[2 * C * LK];  // K e^{G-G0}, then W, then dW
    __shared__ __attribute__((aligned(16))) __bf16 bB[2 * C * LM];  // Q e^{G-G0}, then U
    __shared__ __attribute__((aligned(16))) __bf16 bC[2 * C * LM];  // K e^{G0-G}, then dU
    __shared__ __attribute__((aligned(16))) __bf16 bX[2 * C * LK];  // K e^G
    __shared__ __attribute__((aligned(16))) __bf16 bH[2 * C * LK];  // K^ = K e^{G_last - G}
    __shared__ float sP[C * P16], sM[C * P16], sT[C * P16];  // P (strict lower), M (lower), N then T
    __shared__ float sdM[C * P16], sdT[C * P16];              // N^2, N^4 during the solve; dM; dT, then dP
    __shared__ float sGl[DK], sDg[DK], sdb[NW][C], sB[C];

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < NW);  // 256 threads: the range readfirstlane hides
    const int n = blockIdx.x, bh = blockIdx.y, NC = T / C;
    const size_t t0 = (size_t)bh * T + (size_t)n * C;  // first token row of the chunk
    const float *Sg = states + ((size_t)bh * NC + n) * DV * DK;
    const float *Dg = dstates + ((size_t)bh * NC + n) * DV * DK;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // ---------------------------------------------------------------- loads
    // Inputs first (one 16-byte unit of q, k, a, v, dout per thread), then this wave's state
    // columns (for dQ~ and dW) and rows (for U); nothing waits until it is used.  The two reads
    // of the state (and later the two of dS') are issued together, so that the second finds the
    // lines the first brought into L2.
    const int rk = tid / (DK / 8), ck = 8 * (tid % (DK / 8));
    const int rv = tid / (DV / 8), cv = 8 * (tid % (DV / 8));
    const bool hk = UK == NTH || tid < UK, hv = UV == NTH || tid < UV;
    uint4 xq = {0, 0, 0, 0}, xk = xq, xa = xq, xv = xq, xo = xq;
    if (hk) {
        xq = reinterpret_cast<const uint4 *>(q + t0 * DK)[tid];
        xk = reinterpret_cast<const uint4 *>(k + t0 * DK)[tid];
        xa = reinterpret_cast<const uint4 *>(a + t0 * DK)[tid];
    }
    if (hv) {
        xv = reinterpret_cast<const uint4 *>(v + t0 * DV)[tid];
        xo = reinterpret_cast<const uint4 *>(dout + t0 * DV)[tid];
    }
    const float bv = tid < C ? (float)beta[t0 + tid] : 0.f;
    float scol[TK][NBV][8], srow[TV][NBK][8];
#pragma unroll
    for (int t = 0; t < TK; ++t) load_cols<DK, DV>(Sg, 16 * (wave + NW * t), lane, scol[t]);
#pragma unroll
    for (int t = 0; t < TV; ++t) load_rows<DK>(Sg, 16 * (wave + NW * t), lane, srow[t]);

    if (hk) {
        *reinterpret_cast<uint4 *>(sQ + rk * LK + ck) = xq;
        *reinterpret_cast<uint4 *>(sK + rk * LK + ck) = xk;
        *reinterpret_cast<uint4 *>(sA + rk * LK + ck) = xa;
        const __bf16 *pa = reinterpret_cast<const __bf16 *>(&xa);
        *reinterpret_cast<f32x4 *>(sG + rk * LG + ck) = f32x4{(float)pa[0], (float)pa[1], (float)pa[2], (float)pa[3]};
        *reinterpret_cast<f32x4 *>(sG + rk * LG + ck + 4) = f32x4{(float)pa[4], (float)pa[5], (float)pa[6], (float)pa[7]};
    }
    if (hv) {
        *reinterpret_cast<uint4 *>(sV + rv * LV + cv) = xv;
        *reinterpret_cast<uint4 *>(sO + rv * LV + cv) = xo;
    }
    if (tid < C) sB[tid] = bv;
    __syncthreads();

    // ---------------------------------------------------------------- gate, prefix sum
    if (tid < DK) {  // one branch on the gate form for the whole scan, not one per row
        auto scan = [&](auto ls) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < C; ++r) {
                acc += gate_log2_t<decltype(ls)::value>(sG[r * LG + tid], gmin2);
                sG[r * LG + tid] = acc;
            }
        };
        if (logsig) scan(std::true_type{});
        else scan(std::false_type{});
    }
    __syncthreads();

    // ---------------------------------------------------------------- shared operands
    // Factors as in the chunk form (G in log2 units): Ep = e^{G_r - G_0}, Em = e^{G_0 - G_r},
    // EG = e^{G_r}, EH = e^{G_last - G_r}.
    if (hk) {
        const __bf16 *pq = reinterpret_cast<const __bf16 *>(&xq), *pk = reinterpret_cast<const __bf16 *>(&xk);
        float kp[8], qp[8], km[8], kx[8], kh[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = ck + i;
            const float G = sG[rk * LG + c], G0 = sG[c], Gl = sG[(C - 1) * LG + c];
            const float ep = ex2(G - G0), em = ex2(G0 - G), eg = ex2(G), eh = ex2(Gl - G);
            const float kv = (float)pk[i], qv = (float)pq[i];
            kp[i] = kv * ep;
            qp[i] = qv * ep;
            km[i] = kv * em;
            kx[i] = kv * eg;
            kh[i] = kv * eh;
        }
        st_hl8<LK>(bA, rk, ck, kp);
        st_hl8<LM>(bB, rk, ck, qp);
        st_hl8<LM>(bC, rk, ck, km);
        st_hl8<LK>(bX, rk, ck, kx);
        st_hl8<LK>(bH, rk, ck, kh);
    }
    __syncthreads();

    // ---------------------------------------------------------------- P, T (wave 0); M (wave 1)
    if (wave == 0) {
        const f32x4 p = mm_rows<NBK, LK, LM, true, true>(zero, bA, bC, lane);  // (K Ep)(K Em)^T
        f32x4 nn;  // N = diag(beta) strict_tril(P), as an accumulator tile
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float pv = l16 < r ? p[i] : 0.f;
            sP[r * P16 + l16] = pv;
            nn[i] = sB[r] * pv;
            sT[r * P16 + l16] = nn[i];
        }
        // T = (I - N)(I + N^2)(I + N^4)(I + N^8); the LDS copies are this wave's own writes,
        // which its later reads see once the writes have completed.
        __builtin_amdgcn_s_waitcnt(0xc07f);
        auto rowsN = [&](const float *X) { return [X, l16 = l16, g = g](int i) { return X[l16 * P16 + 4 * g + i]; }; };
        const f32x4 n2 = mm16(zero, rowsN(sT), [&](int i) { return nn[i]; });
#pragma unroll
        for (int i = 0; i < 4; ++i) sdM[(4 * g + i) * P16 + l16] = n2[i];
        __builtin_amdgcn_s_waitcnt(0xc07f);
        const f32x4 n4 = mm16(zero, rowsN(sdM), [&](int i) { return n2[i]; });
#pragma unroll
        for (int i = 0; i < 4; ++i) sdT[(4 * g + i) * P16 + l16] = n4[i];
        __builtin_amdgcn_s_waitcnt(0xc07f);
        const f32x4 n8 = mm16(zero, rowsN(sdT), [&](int i) { return n4[i]; });
        f32x4 r1;
#pragma unroll
        for (int i = 0; i < 4; ++i) r1[i] = n4[i] + n8[i] + ((4 * g + i) == l16 ? 1.f : 0.f);
        r1 = mm16(r1, rowsN(sdT), [&](int i) { return n8[i]; });   // + N^4 N^8
        const f32x4 r2 = mm16(r1, rowsN(sdM), [&](int i) { return r1[i]; });  // (I + N^2) R1
        const f32x4 nr = mm16(zero, rowsN(sT), [&](int i) { return r2[i]; });  // N R2
#pragma unroll
        for (int i = 0; i < 4; ++i) sT[(4 * g + i) * P16 + l16] = r2[i] - nr[i];
    } else if (wave == 1) {
        const f32x4 m = mm_rows<NBK, LM, LM, true, true>(zero, bB, bC, lane);  // (Q Ep)(K Em)^T
#pragma unroll
        for (int i = 0; i < 4; ++i) sM[(4 * g + i) * P16 + l16] = l16 <= 4 * g + i ? m[i] : 0.f;
    }

    // ---------------------------------------------------------------- dQ~ = dO S^T
    f32x4 dQa[TK], dKa[TK], dGa[TK], dUa[TV];  // this wave's key tiles of dq, dk, dG; value tiles of dU
    HL8 scs[TK][NBV];                            // state columns, split, kept for dW
#pragma unroll
    for (int t = 0; t < TK; ++t) {
        const int c = 16 * (wave + NW * t) + l16;
#pragma unroll
        for (int b = 0; b < NBV; ++b) scs[t][b] = split8(scol[t][b]);
        const f32x4 acc = mm_h_reg<NBV, LV>(zero, sO, scs[t], lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            dQa[t][i] = acc[i] * ex2(sG[r * LG + c]);          // dQ~ e^G
            dGa[t][i] = (float)sQ[r * LK + c] * dQa[t][i];     // dQ~ * Q~
            dKa[t][i] = 0.f;
        }
        asm volatile("" : "+v"(dQa[t]), "+v"(dGa[t]));  // formed here, not where they are next used
    }
    __syncthreads();  // T and M are in; the P, M operand blocks are free

    // ---------------------------------------------------------------- W = T diag(b) K e^G, U~ = T diag(b) V
    auto tb = [&](int i) { return sT[l16 * P16 + 4 * g + i] * sB[4 * g + i]; };  // (T diag(b))[m][4g+i]
#pragma unroll
    for (int t = 0; t < TK; ++t) {
        const int c = 16 * (wave + NW * t) + l16;
        const f32x4 w = mm16(zero, tb, [&](int i) {
            const int s = 4 * g + i;
            return (float)bX[s * LK + c] + (float)bX[16 * LK + s * LK + c];
        });
        st_acc_hl<LK>(bA, w, 16 * (wave + NW * t), lane);
    }
    f32x4 Ua[TV];
#pragma unroll
    for (int t = 0; t < TV; ++t) {
        const int j = 16 * (wave + NW * t) + l16;
        Ua[t] = mm16(zero, tb, [&](int i) { return (float)sV[(4 * g + i) * LV + j]; });
    }
    __syncthreads();  // W is in

    // ---------------------------------------------------------------- U = U~ - W S, dU = K^ dS' + M^T dO
#pragma unroll
    for (int t = 0; t < TV; ++t) {
        const int j0 = 16 * (wave + NW * t);
        HL8 srs[NBK];
#pragma unroll
        for (int b = 0; b < NBK; ++b) srs[b] = split8(srow[t][b]);
        const f32x4 ws = mm_hl_reg<NBK, LK>(zero, bA, srs, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) Ua[t][i] -= ws[i];
        st_acc_hl<LM>(bB, Ua[t], j0, lane);
    }
    // dS' rows (for K^ dS') and then its columns (for dK^, dgamma), each where the registers of
    // the previous block are free; the scheduling barriers keep the compiler from hoisting them.
    __builtin_amdgcn_sched_barrier(0);
    float drow[TV][NBK][8];
#pragma unroll
    for (int t = 0; t < TV; ++t) load_rows<DK>(Dg, 16 * (wave + NW * t), lane, drow[t]);
#pragma unroll
    for (int t = 0; t < TV; ++t) {
        const int j0 = 16 * (wave + NW * t);
        HL8 drs[NBK];
#pragma unroll
        for (int b = 0; b < NBK; ++b) drs[b] = split8(drow[t][b]);
        dUa[t] = mm_hl_reg<NBK, LK>(zero, bH, drs, lane);
        dUa[t] = mm16(dUa[t], [&](int i) { return sM[(4 * g + i) * P16 + l16]; },
                      [&](int i) { return (float)sO[(4 * g + i) * LV + j0 + l16]; });
        st_acc_hl<LM>(bC, dUa[t], j0, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    float dcol[TK][NBV][8];  // dS' columns of this wave's key tiles, for dK^ and dgamma
#pragma unroll
    for (int t = 0; t < TK; ++t) load_cols<DK, DV>(Dg, 16 * (wave + NW * t), lane, dcol[t]);
    __syncthreads();  // U, dU are in; W is free

    // ---------------------------------------------------------------- dW = -dU S^T, dX, dY, dM
    float db[4] = {0.f, 0.f, 0.f, 0.f};  // this wave's part of dbeta for rows 4g+i
    auto tt = [&](int i) { return sT[(4 * g + i) * P16 + l16]; };  // T^T[m][4g+i]
#pragma unroll
    for (int t = 0; t < TK; ++t) {
        const int c0 = 16 * (wave + NW * t), c = c0 + l16;
        f32x4 dw = mm_hl_reg<NBV, LM>(zero, bC, scs[t], lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) dw[i] = -dw[i];
        st_acc_hl<LK>(bA, dw, c0, lane);
        const f32x4 dx = mm16(zero, tt, [&](int i) { return dw[i]; });  // dX = T^T dW
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float eg = ex2(sG[r * LG + c]), kt = (float)sK[r * LK + c] * eg;
            dKa[t][i] += sB[r] * dx[i] * eg;  // b dX e^G
            dGa[t][i] += sB[r] * dx[i] * kt;  // b dX * K~
            db[i] += dx[i] * kt;
        }
    }
#pragma unroll
    for (int t = 0; t < TV; ++t) {
        const int j = 16 * (wave + NW * t) + l16;
        const f32x4 dy = mm16(zero, tt, [&](int i) { return dUa[t][i]; });  // dY = T^T dU
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            dv[(t0 + r) * DV + j] = sB[r] * dy[i];
            db[i] += dy[i] * (float)sV[r * LV + j];
        }
    }
    if (wave == NW - 1) {  // dM = tril(dO U^T)
        const f32x4 m = mm_rows<NBV, LV, LM, false, true>(zero, sO, bB, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdM[(4 * g + i) * P16 + l16] = l16 <= 4 * g + i ? m[i] : 0.f;
    }
    // dK^ = U dS'^T and dgamma = sum over values of S * dS'
#pragma unroll
    for (int t = 0; t < TK; ++t) {
        const int c = 16 * (wave + NW * t) + l16;
        HL8 dcs[NBV];
        float dgam = 0.f;
#pragma unroll
        for (int b = 0; b < NBV; ++b) {
            dcs[b] = split8(dcol[t][b]);
            // S and dS' as hi + lo; the empty asm makes the compiler widen the 16-bit values
            // again instead of keeping the 32-bit forms of the splits alive
            HL8 sv = scs[t][b], dw = dcs[b];
            asm volatile("" : "+v"(sv.h), "+v"(sv.l), "+v"(dw.h), "+v"(dw.l));
#pragma unroll
            for (int s = 0; s < 8; ++s) dgam += ((float)sv.h[s] + (float)sv.l[s]) * ((float)dw.h[s] + (float)dw.l[s]);
        }
        const f32x4 dkh = mm_hl_reg<NBV, LM>(zero, bB, dcs, lane);
        const float Gl = sG[(C - 1) * LG + c];
        float col = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float eh = ex2(Gl - sG[r * LG + c]), kh = (float)sK[r * LK + c] * eh;
            dKa[t][i] += dkh[i] * eh;  // dK^ e^{G_last - G}
            dGa[t][i] -= dkh[i] * kh;  // - dK^ * K^
            col += dkh[i] * kh;
        }
        col += __shfl_xor(col, 16, 64);
        col += __shfl_xor(col, 32, 64);
        dgam += __shfl_xor(dgam, 16, 64);
        dgam += __shfl_xor(dgam, 32, 64);
        if (g == 0) {
            sGl[c] = col;   // sum over the chunk's rows of dK^ * K^
            sDg[c] = dgam;  // dgamma_c
        }
    }
    __syncthreads();  // dW, dM are in

    // ---------------------------------------------------------------- dT, dA, dP (wave 0)
    if (wave == 0) {
        // dT[r][s] = b_s (sum_c dW[r][c] (K e^G)[s][c] + sum_j dU[r][j] V[s][j])
        f32x4 d = mm_rows<NBK, LK, LK, true, true>(zero, bA, bX, lane);
        d = mm_rows<NBV, LM, LV, true, false>(d, bC, sV, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdT[(4 * g + i) * P16 + l16] = d[i] * sB[l16];
        __builtin_amdgcn_s_waitcnt(0xc07f);
        // dA = -strict_tril(T^T dT T^T): z = dT T^T, then T^T z
        const f32x4 z = mm16(zero, [&](int i) { return sdT[l16 * P16 + 4 * g + i]; },
                             [&](int i) { return sT[l16 * P16 + 4 * g + i]; });
        const f32x4 w = mm16(zero, tt, [&](int i) { return z[i]; });
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float dpa = l16 < r ? -w[i] : 0.f;
            db[i] += dpa * sP[r * P16 + l16];
            sdT[r * P16 + l16] = sB[r] * dpa;  // dP = diag(b) dA, over dT
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // sum over the 16 columns this lane group holds
        float s = db[i];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        s += __shfl_xor(s, 8, 64);
        if (l16 == 0) sdb[wave][4 * g + i] = s;
    }
    __syncthreads();  // dP is in

    // ---------------------------------------------------------------- pairwise terms of M and P, outputs
    // The 16-deep B operands are this lane's own rows 4g+i of its column, as are the outputs.
    float *sdg = reinterpret_cast<float *>(bX);  // dG [C][LG], K e^G no longer needed
    const HL4 dMa = split_at([&](int i) { return sdM[l16 * P16 + 4 * g + i]; });    // dM
    const HL4 dMb = split_at([&](int i) { return sdM[(4 * g + i) * P16 + l16]; });  // dM^T
    const HL4 dPa = split_at([&](int i) { return sdT[l16 * P16 + 4 * g + i]; });    // dP
    const HL4 dPb = split_at([&](int i) { return sdT[(4 * g + i) * P16 + l16]; });  // dP^T
#pragma unroll
    for (int t = 0; t < TK; ++t) {
        const int c = 16 * (wave + NW * t) + l16;
        const float G0 = sG[c], Gl = sG[(C - 1) * LG + c];
        float ep[4], em[4], kr[4], qr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float G = sG[r * LG + c];
            ep[i] = ex2(G - G0);
            em[i] = ex2(G0 - G);
            kr[i] = (float)sK[r * LK + c];
            qr[i] = (float)sQ[r * LK + c];
        }
        const HL4 km = split_at([&](int i) { return kr[i] * em[i]; });
        const f32x4 x1 = mm16_hl(zero, dMa, km);                                                // dM Km
        const f32x4 x2 = mm16_hl(zero, dMb, split_at([&](int i) { return qr[i] * ep[i]; }));  // dM^T Qp
        const f32x4 x3 = mm16_hl(zero, dPa, km);                                                // dP Km
        const f32x4 x4 = mm16_hl(zero, dPb, split_at([&](int i) { return kr[i] * ep[i]; }));  // dP^T Kp
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            const float a1 = x1[i] * ep[i], a2 = x2[i] * em[i], a3 = x3[i] * ep[i], a4 = x4[i] * em[i];
            const float dqv = dQa[t][i] + a1, dkv = dKa[t][i] + a2 + a3 + a4;
            float dg = dGa[t][i] + qr[i] * a1 - kr[i] * a2 + kr[i] * a3 - kr[i] * a4;
            if (r == C - 1) dg += sGl[c] + sDg[c] * ex2(Gl);  // G_last: K^ and gamma
            dq[(t0 + r) * DK + c] = dqv;
            dk[(t0 + r) * DK + c] = dkv;
            sdg[r * LG + c] = dg;
        }
    }
    __syncthreads();
    if (tid < DK) {  // dg = reverse prefix sum of dG down the chunk, da = dg g'(a)
        float acc = 0.f;
#pragma unroll
        for (int r = C - 1; r >= 0; --r) {
            const float av = (float)sA[r * LK + tid], sg = 1.f / (1.f + __expf(-av));
            acc += sdg[r * LG + tid];
            da[(t0 + r) * DK + tid] = acc * (logsig ? (1.f - sg) : gmin * sg * (1.f - sg));
        }
    }
    if (tid < C) {
        float sb = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sb += sdb[w][tid];
        dbeta[t0 + tid] = sb;
    }
}

}  // namespace kda
