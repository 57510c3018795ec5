// Backward pass of the chunked forward: gradients of
//   L = sum_t dout_t . o_t + <dfinal, S_T>
// with respect to q, k, v, a, beta and the initial state, for training ("Breaking
// Through Trillion-Parameter Multimodal MoE ...", sec. 2.1: the operator change must be
// invisible to the training scripts above it, so it must supply exactly these gradients).
//
// The chunk form, with 16-token chunks (the gradients are those of the function, so the
// backward chooses its own chunk; one 16-row tile per chunk needs a single Gamma reference,
// the chunk's first row, within the range the bound guarantees).  With S = state^T (dk x
// dv), per chunk (G the chunk's inclusive log-cumsum, E_rs = e^{G_r - G_s} per channel):
//   forward, recomputed:  A = strict_tril(diag(b) P),  P_rs = sum_c k_rc k_sc E_rsc,
//     M = tril(sum_c q_rc k_sc E_rsc),  T = (I + A)^-1,  W = T diag(b) K e^G,
//     U = T diag(b) V - W S,  K^ = K e^{G_last - G},  gamma = e^{G_last}
//   reverse over chunks (dS' = dL/d(state at the chunk's end), kda_bwd_dstate_kernel):
//     dS = diag(gamma) dS' + Qbar^T dO - W^T (K^ dS'),   Qbar = Q e^G - M W
//   per chunk, in parallel (kda_bwd_chunk_kernel):
//     dU = M^T dO + K^ dS'   dQ~ = dO S^T   dK^ = U dS'^T   dW = -dU S^T   dM = tril(dO U^T)
//     dgamma = rowsum(S * dS')   dT = dW (b K e^G)^T + dU (b V)^T   dX = T^T dW   dY = T^T dU
//     dA = -strict_tril(T^T dT T^T)   dv = b dY   dbeta = rowsum(dX K e^G + dY V + dA P)
//     and the pairwise terms of M and P into dq, dk and dG, then dg = reverse cumsum of dG.
// Every product runs on fp32 MFMA (16x16x4), operands read through index functions.
#pragma once
#include "kda_device.h"
#include "kda_layout.h"

namespace kda {

// 16x16x16 bf16 MFMA: lane (g, m) supplies A[m][4 g .. 4 g + 3] and lane (g, n) B[4 g .. 4 g + 3][n],
// which is where an accumulator tile holds rows 4 g .. 4 g + 3 of column n.
__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

// x = hi + lo in bf16 (about 16 significand bits, the full fp32 range), two values per packed
// conversion.  V: float[4] or f32x4.
template <typename V>
__device__ __forceinline__ void split4(const V &x, bf16x4 &h, bf16x4 &l) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const f32x2 v = {x[2 * p], x[2 * p + 1]};
        const bf16x2 hp = __builtin_convertvector(v, bf16x2);
        const bf16x2 lp = __builtin_convertvector(v - __builtin_convertvector(hp, f32x2), bf16x2);
        h[2 * p] = hp[0];
        h[2 * p + 1] = hp[1];
        l[2 * p] = lp[0];
        l[2 * p + 1] = lp[1];
    }
}

// acc += A (16 x K) B (K x 16) on fp32 MFMA: A(m, k) and B(k, n) return A[m][k] and B[k][n]
// (m, n in 0..15).  In v_mfma_f32_16x16x4f32 lane l supplies A[l%16][k0 + l/16] and
// B[k0 + l/16][l%16]; acc[i] is D[4 (l/16) + i][l%16].
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma_tile(f32x4 acc, const FA &A, const FB &B, int lane) {
    const int m = lane & 15, kq = lane >> 4;
#pragma unroll 8
    for (int k0 = 0; k0 < K; k0 += 4)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(A(m, k0 + kq), B(k0 + kq, m), acc, 0, 0, 0);
    return acc;
}

// The same product with bf16 hi + lo operands: x = hi + lo with hi = bf16(x), lo = bf16(x - hi)
// (about 16 significand bits, the full fp32 range), three 16x16x32 MFMAs per 32-deep block
// (hi hi, lo hi, hi lo).  This product is private to the tile, so its K slots are its own:
// slot j of lane group g is k = k0 + 8 g + j.  K a multiple of 16 (a half block is padded
// with zeros).
template <int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma_tile_split(f32x4 acc, const FA &A, const FB &B, int lane) {
    const int m = lane & 15, g8 = 8 * (lane >> 4);
    static_assert(K % 16 == 0, "K in 16-deep steps");
#pragma unroll 2
    for (int k0 = 0; k0 < K; k0 += 32) {
        bf16x8 ah, al, bh, bl;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int kk = k0 + g8 + j;
            const bool in = (K % 32 == 0) || kk < K;
            const float x = in ? A(m, kk) : 0.f, y = in ? B(kk, m) : 0.f;
            ah[j] = (__bf16)x;
            al[j] = (__bf16)(x - (float)ah[j]);
            bh[j] = (__bf16)y;
            bl[j] = (__bf16)(y - (float)bh[j]);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
    }
    return acc;
}

// The products of the chunk-parallel stage over a dk- or dv-deep dimension: fp32 for fp32
// inputs (their 1e-4 bar), bf16 hi + lo otherwise.
template <bool F32, int K, typename FA, typename FB>
__device__ __forceinline__ f32x4 mma_big(f32x4 acc, const FA &A, const FB &B, int lane) {
    if constexpr (F32) return mma_tile<K>(acc, A, B, lane);
    else return mma_tile_split<K>(acc, A, B, lane);
}

// Element (r, c) of a stored tile-pair block (kda_layout.h): tiles of 16 x 16 in
// accumulator order, the two tiles of a pair interleaved per lane.  `pairs_along_rows`:
// the pair joins tile rows 2p and 2p+1 (K^), else tile columns (W^T, Qbar^T stored with
// pairs along dk, their row dimension).  ntc: tiles per row of the block's tile grid in the
// stored order (NT for W^T/Qbar^T, NDK for K^).
__device__ __forceinline__ int pair_offset(int r, int c, int ntc) {
    // a block X stored as pairs [r/32][c/16]: pair (tile rows 2p, 2p+1) for tile column c/16
    const int tr = r >> 4, tc = c >> 4, rr = r & 15, cc = c & 15;
    return (((tr >> 1) * ntc + tc) * 64 + 16 * (rr >> 2) + cc) * 8 + 4 * (tr & 1) + (rr & 3);
}

template <int DK, int DV, bool F32>
struct BwdCfg {
    using E = typename std::conditional<F32, float, __bf16>::type;
    using OH = typename std::conditional<F32, float, _Float16>::type;  // record operand type
    static constexpr int C = 16;
    static constexpr KdaLayout L = kda_layout(C, DK, DV, sizeof(E));
    static constexpr int NS = DV / 16;
};

// ---------------------------------------------------------------------------------------
// Reverse pass over the chunks of one head and one 16-wide value slice: carries the slice of
// dS' (dk x 16, fp32) from the last chunk to the first, storing it for every chunk (the
// gradient of the state that chunk ends in), and gives dL/dS_0 at the end.  Reads W^T, Qbar^T,
// K^ and gamma from the chunk records of the forward's chunk stage (16-token chunks) and the
// chunk's 16 x 16 block of dout.
// Work-group = 5 waves: waves 0-3 compute (P = K^ dS' split over the key dimension, then each
// wave's dk tiles of the update), wave 4 streams each chunk's record and dout block into a ring
// of three LDS slots with direct global->LDS loads, two chunks ahead; it alone waits on its
// memory counter, so the barriers only order LDS traffic.
template <int DK, int DV, bool F32>
__global__ __launch_bounds__(320) void kda_bwd_dstate_kernel(
    const unsigned char *__restrict__ ws, const typename BwdCfg<DK, DV, F32>::E *__restrict__ dout,
    const float *__restrict__ dfinal, int T, int BH, float *__restrict__ dstates, float *__restrict__ dinit)
{
    using Cfg = BwdCfg<DK, DV, F32>;
    using E = typename Cfg::E;
    using OH = typename Cfg::OH;
    constexpr KdaLayout L = Cfg::L;
    constexpr int NS = Cfg::NS, NDK = DK / 16, NTW = (NDK + 3) / 4;  // dk tiles per compute wave
    constexpr int R1 = (int)L.region1, NU = (R1 + 15) / 16;          // 16-byte units of region 1
    constexpr int NBLK = (NU + 63) / 64;                              // 1 KiB direct-load blocks
    constexpr int RB = NBLK * 1024, SLOT = RB + 1024;                 // record + dout block
    constexpr int NDMA = NBLK + 1;                                    // loader instructions per chunk
    static_assert(NDMA <= 63, "partial wait needs the count in the vmcnt field");
    constexpr int PD = 17;

    __shared__ __attribute__((aligned(1024))) unsigned char sRing[3 * SLOT];
    __shared__ float sD[DK * PD];       // dS' slice: [key c][value j]
    __shared__ float sPp[4][16 * PD];   // split-K partials of P = K^ dS'

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < 5);  // 320 threads: the range readfirstlane hides
    // all slices of a head on one XCD (work-group ids are dealt round-robin to the 8 XCDs), so
    // that the slices' reads of the same chunk record meet in that XCD's L2
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int bh = (local / NS) * 8 + xcd, slice = local % NS, j0 = 16 * slice;
    if (bh >= BH) return;
    const int NC = T / 16;
    const unsigned char *rec0 = ws + (size_t)bh * NC * L.stride;

    // loader: chunk n into slot s (every lane of every instruction loads; the last block's spare
    // lanes re-read the last unit into the slot's padding)
    auto issue = [&](int n, int s) {
        const unsigned char *src = rec0 + (size_t)n * L.stride;
        lds_u8 *dst = lds_base(sRing) + s * SLOT;
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
            const int u = min(blk * 64 + lane, NU - 1);
            __builtin_amdgcn_global_load_lds(src + (size_t)u * 16, (lds_void *)(dst + blk * 1024), 16, 0, 0);
        }
        // dout block: 16 rows x 16 values of this slice, 16 bytes per lane
        constexpr int LPR = 16 * (int)sizeof(E) / 16;  // lanes per row (2 or 4)
        const int row = min(lane / LPR, 15), part = lane % LPR;
        const unsigned char *srow = reinterpret_cast<const unsigned char *>(
            dout + ((size_t)bh * T + (size_t)n * 16 + row) * DV + j0);
        __builtin_amdgcn_global_load_lds(srow + 16 * part, (lds_void *)(dst + RB), 16, 0, 0);
    };

    // dS' of the last chunk: dfinal (or zero), kept in registers in accumulator order
    f32x4 D[NTW];
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int mt = wave + 4 * x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * mt + 4 * g + i;
            D[x][i] = (wave < 4 && mt < NDK && dfinal != nullptr) ? dfinal[((size_t)bh * DV + j0 + l16) * DK + c] : 0.f;
        }
    }
    if (wave == 4 && NC > 0) {
        issue(NC - 1, 0);
        if (NC > 1) {
            issue(NC - 2, 1);
            wait_vmcnt<NDMA>();
        } else {
            wait_vmcnt<0>();
        }
    }

    for (int it = 0; it < NC; ++it) {
        const int n = NC - 1 - it;
        const unsigned char *cur = sRing + (it % 3) * SLOT;
        barrier_lds();  // (A) chunk n's slot has landed; the previous chunk is done with sD and sPp
        if (wave < 4) {
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                const int mt = wave + 4 * x;
                if (mt >= NDK) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) sD[(16 * mt + 4 * g + i) * PD + l16] = D[x][i];
                // dS' of this chunk's end, for the chunk-parallel stage: dstates[bh][n][value][key]
                *reinterpret_cast<f32x4 *>(dstates + (((size_t)bh * NC + n) * DV + j0 + l16) * DK + 16 * mt + 4 * g) = D[x];
            }
        }
        barrier_lds();  // (B) sD holds dS'
        const OH *rWT = reinterpret_cast<const OH *>(cur + L.wt);
        const OH *rQB = reinterpret_cast<const OH *>(cur + L.qbt);
        const OH *rKH = reinterpret_cast<const OH *>(cur + L.kh);
        const float *rG = reinterpret_cast<const float *>(cur + L.gam);
        const int *rS = reinterpret_cast<const int *>(cur + L.scl);
        const E *rdO = reinterpret_cast<const E *>(cur + RB);  // [row][16]
        if (wave == 4) {
            if (it + 2 < NC) issue(n - 2, (it + 2) % 3);
        } else {  // P = K^ dS' (16 x 16), the key dimension split over the four waves
            constexpr int KW = DK / 4;
            const int c0 = KW * wave;
            const float fK = ldexp2(1.f, -rS[2]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma_tile<KW>(acc,
                               [&](int m, int kk) { return (float)rKH[pair_offset(m, c0 + kk, NDK)] * fK; },
                               [&](int kk, int nn) { return sD[(c0 + kk) * PD + nn]; }, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sPp[wave][(4 * g + i) * PD + l16] = acc[i];
        }
        barrier_lds();  // (C) the partials of P are in
        if (wave == 4) {
            if (it + 2 < NC) wait_vmcnt<NDMA>();  // chunk n - 1 has landed (n - 2 may be in flight)
            else wait_vmcnt<0>();
        } else {
            // dS = diag(gamma) dS' + Qbar^T dO - W^T P  (rows c of this wave's dk tiles)
            const float fW = ldexp2(1.f, -rS[0]), fQ = ldexp2(1.f, -rS[1]);
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                const int mt = wave + 4 * x;
                if (mt >= NDK) continue;
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = rG[16 * mt + 4 * g + i] * D[x][i];
                acc = mma_tile<16>(acc, [&](int m, int kk) { return (float)rQB[pair_offset(16 * mt + m, kk, 1)] * fQ; },
                                   [&](int kk, int nn) { return to_f(rdO[kk * 16 + nn]); }, lane);
                acc = mma_tile<16>(acc, [&](int m, int kk) { return -(float)rWT[pair_offset(16 * mt + m, kk, 1)] * fW; },
                                   [&](int kk, int nn) {
                                       const int o = kk * PD + nn;
                                       return (sPp[0][o] + sPp[1][o]) + (sPp[2][o] + sPp[3][o]);
                                   },
                                   lane);
                D[x] = acc;
            }
        }
    }
    if (dinit != nullptr && wave < 4) {
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int mt = wave + 4 * x;
            if (mt >= NDK) continue;
            *reinterpret_cast<f32x4 *>(dinit + ((size_t)bh * DV + j0 + l16) * DK + 16 * mt + 4 * g) = D[x];
        }
    }
}

// ---------------------------------------------------------------------------------------
// Gradients of one 16-token chunk of one head, from the state it starts from (states) and
// the gradient of the state it ends in (dstates).  All intermediates in fp32; the state S
// is held in LDS, dS' is staged through LDS a quarter at a time.  Work-group = 8 waves
// (two per SIMD, the LDS allows one work-group per CU); products over a dk- or dv-wide
// dimension are split by 16-column tiles over the waves, and each wave keeps its tiles of
// dq, dk and dG in registers.
template <int DK, int DV, bool F32>
__global__ __launch_bounds__(512, 1) void kda_bwd_chunk_kernel(
    const typename BwdCfg<DK, DV, F32>::E *__restrict__ q, const typename BwdCfg<DK, DV, F32>::E *__restrict__ k,
    const typename BwdCfg<DK, DV, F32>::E *__restrict__ v, const typename BwdCfg<DK, DV, F32>::E *__restrict__ a,
    const typename BwdCfg<DK, DV, F32>::E *__restrict__ beta,
    const typename BwdCfg<DK, DV, F32>::E *__restrict__ dout, float gmin2, float gmin, int logsig, int T,
    const float *__restrict__ states, const float *__restrict__ dstates, float *__restrict__ dq,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ da, float *__restrict__ dbeta)
{
    constexpr int C = 16, PK = DK + 1, PV = DV + 1, P16 = 17, NW = 8, NTH = 64 * NW;
    constexpr int NDK = DK / 16, NDV = DV / 16, NTK = (NDK + NW - 1) / NW, NTV = (NDV + NW - 1) / NW;
    __shared__ float sQ[C * PK], sK[C * PK], sG[C * PK], sV[C * PV], sdO[C * PV];
    __shared__ float sS[DV * PK];  // the chunk's start state as stored: [value j][key c]
    __shared__ float sW[C * PK];   // W, then dW, then dG
    __shared__ float sU[C * PV];   // U~, then U
    __shared__ float sdU[C * PV];  // K^ dS', then dU
    __shared__ float sP[C * P16], sM[C * P16], sT[C * P16], sdM[C * P16], sdT[C * P16], sdA[C * P16];
    __shared__ float sB[C], sGl[DK], sDg[DK], sdb[NW][C];
    __shared__ float sDq[DV / 4 * PK];  // a quarter of dS' (value rows) at a time

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < 8);  // 512 threads: the range readfirstlane hides
    const int n = blockIdx.x, bh = blockIdx.y, NC = T / C;
    const size_t t0 = (size_t)bh * T + (size_t)n * C;  // first token row of the chunk
    const float *Sg = states + ((size_t)bh * NC + n) * DV * DK;
    const float *Dg = dstates + ((size_t)bh * NC + n) * DV * DK;  // dS' as [value j][key c]

    // ---------------------------------------------------------------- loads, G
    // Every load of the chunk is issued before any is consumed (16-byte accesses; a chunk's
    // rows of q, k, v, dout and a are contiguous, as is its state), so the work-group pays one
    // memory round trip; a goes to LDS (its gate and prefix sum are taken from there).
    {
        using E = typename BwdCfg<DK, DV, F32>::E;
        constexpr int VE = 16 / (int)sizeof(E);                       // elements per 16 bytes
        constexpr int UK = C * DK / VE, UV = C * DV / VE;             // 16-byte units per block
        constexpr int NK = (UK + NTH - 1) / NTH, NV = (UV + NTH - 1) / NTH, NSS = DV * DK / 4 / NTH;
        uint4 xq[NK], xk[NK], xa[NK], xv[NV], xo[NV];
        f32x4 xs[NSS];
        const uint4 *gq = reinterpret_cast<const uint4 *>(q + t0 * DK);
        const uint4 *gk = reinterpret_cast<const uint4 *>(k + t0 * DK);
        const uint4 *ga = reinterpret_cast<const uint4 *>(a + t0 * DK);
        const uint4 *gv = reinterpret_cast<const uint4 *>(v + t0 * DV);
        const uint4 *go = reinterpret_cast<const uint4 *>(dout + t0 * DV);
#pragma unroll
        for (int x = 0; x < NSS; ++x) xs[x] = reinterpret_cast<const f32x4 *>(Sg)[tid + NTH * x];
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int u = min(tid + NTH * x, UK - 1);
            xq[x] = gq[u];
            xk[x] = gk[u];
            xa[x] = ga[u];
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int u = min(tid + NTH * x, UV - 1);
            xv[x] = gv[u];
            xo[x] = go[u];
        }
        const float bv = to_f(beta[t0 + (tid & (C - 1))]);
#pragma unroll
        for (int x = 0; x < NSS; ++x) {
            const int e = 4 * (tid + NTH * x), j = e / DK, c = e % DK;
#pragma unroll
            for (int i = 0; i < 4; ++i) sS[j * PK + c + i] = xs[x][i];
        }
#pragma unroll
        for (int x = 0; x < NK; ++x) {
            const int u = tid + NTH * x;
            if (u >= UK) continue;
            const int e = u * VE, r = e / DK, c = e % DK;
            const E *pq = reinterpret_cast<const E *>(&xq[x]), *pk = reinterpret_cast<const E *>(&xk[x]);
            const E *pa = reinterpret_cast<const E *>(&xa[x]);
#pragma unroll
            for (int i = 0; i < VE; ++i) {
                sQ[r * PK + c + i] = to_f(pq[i]);
                sK[r * PK + c + i] = to_f(pk[i]);
                sG[r * PK + c + i] = to_f(pa[i]);  // a for now; G below
            }
        }
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const int u = tid + NTH * x;
            if (u >= UV) continue;
            const int e = u * VE, r = e / DV, c = e % DV;
            const E *pv = reinterpret_cast<const E *>(&xv[x]), *po = reinterpret_cast<const E *>(&xo[x]);
#pragma unroll
            for (int i = 0; i < VE; ++i) {
                sV[r * PV + c + i] = to_f(pv[i]);
                sdO[r * PV + c + i] = to_f(po[i]);
            }
        }
        if (tid < C) sB[tid] = bv;
    }
    __syncthreads();
    float gpr[C];  // dg/da of column tid (threads tid < DK), used at the end
    if (tid < DK) {  // gate and prefix sum down the chunk, in place (log2 units); g'(a) kept for da
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < C; ++r) {
            const float av = sG[r * PK + tid];
            acc += gate_log2(av, gmin2, logsig);
            const float sg = 1.f / (1.f + __expf(-av));
            gpr[r] = logsig ? (1.f - sg) : gmin * sg * (1.f - sg);  // dg/da, kept by this thread
            sG[r * PK + tid] = acc;
        }
    }
    __syncthreads();

    // factors (G in log2 units; each at most 1 except Em, at most e^{15 |g_min|})
    auto G = [&](int r, int c) { return sG[r * PK + c]; };
    auto Ep = [&](int r, int c) { return ex2(G(r, c) - G(0, c)); };       // e^{G_r - G_0}
    auto Em = [&](int r, int c) { return ex2(G(0, c) - G(r, c)); };       // e^{G_0 - G_r}
    auto EG = [&](int r, int c) { return ex2(G(r, c)); };                 // e^{G_r}
    auto EH = [&](int r, int c) { return ex2(G(C - 1, c) - G(r, c)); };   // e^{G_last - G_r}
    auto Kv = [&](int r, int c) { return sK[r * PK + c]; };
    auto Qv = [&](int r, int c) { return sQ[r * PK + c]; };

    // ---------------------------------------------------------------- P, M, T
    if (wave == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DK>(acc, [&](int m, int kk) { return Kv(m, kk) * Ep(m, kk); },
                           [&](int kk, int nn) { return Kv(nn, kk) * Em(nn, kk); }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sP[(4 * g + i) * P16 + l16] = (l16 < 4 * g + i) ? acc[i] : 0.f;
    } else if (wave == 1) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DK>(acc, [&](int m, int kk) { return Qv(m, kk) * Ep(m, kk); },
                           [&](int kk, int nn) { return Kv(nn, kk) * Em(nn, kk); }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sM[(4 * g + i) * P16 + l16] = (l16 <= 4 * g + i) ? acc[i] : 0.f;
    }
    __syncthreads();
    if (tid < C) {  // T = (I + A)^-1 by forward substitution, lane = column
        const int j = tid;
        for (int r = 0; r < C; ++r) {
            float x = (r == j) ? 1.f : 0.f;
            for (int u = j; u < r; ++u) x -= sB[r] * sP[r * P16 + u] * sT[u * P16 + j];
            sT[r * P16 + j] = (r < j) ? 0.f : x;
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- W = T X, U~ = T Y
    auto Xv = [&](int r, int c) { return sB[r] * Kv(r, c) * EG(r, c); };  // b K e^G
#pragma unroll
    for (int x = 0; x < NTK; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDK) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_tile<C>(acc, [&](int m, int kk) { return sT[m * P16 + kk]; },
                          [&](int kk, int nn) { return Xv(kk, 16 * nt + nn); }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sW[(4 * g + i) * PK + 16 * nt + l16] = acc[i];
    }
#pragma unroll
    for (int x = 0; x < NTV; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDV) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_tile<C>(acc, [&](int m, int kk) { return sT[m * P16 + kk]; },
                          [&](int kk, int nn) { return sB[kk] * sV[kk * PV + 16 * nt + nn]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sU[(4 * g + i) * PV + 16 * nt + l16] = acc[i];
    }
    __syncthreads();

    // ---------------------------------------------------------------- U = U~ - W S, dQ~ = dO S^T
    f32x4 dQa[NTK], dKa[NTK], dGa[NTK];  // this wave's dk tiles of dq, dk and dG
#pragma unroll
    for (int x = 0; x < NTV; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDV) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DK>(acc, [&](int m, int kk) { return sW[m * PK + kk]; },
                           [&](int kk, int nn) { return sS[(16 * nt + nn) * PK + kk]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float *p = &sU[(4 * g + i) * PV + 16 * nt + l16];
            *p = *p - acc[i];
        }
    }
#pragma unroll
    for (int x = 0; x < NTK; ++x) {
        const int nt = wave + NW * x;
        dQa[x] = dKa[x] = dGa[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (nt >= NDK) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DV>(acc, [&](int m, int kk) { return sdO[m * PV + kk]; },
                           [&](int kk, int nn) { return sS[kk * PK + 16 * nt + nn]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i, c = 16 * nt + l16;
            dQa[x][i] = acc[i] * EG(r, c);        // dQ~ e^G
            dGa[x][i] = Qv(r, c) * dQa[x][i];     // dQ~ * Q~
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- with dS': K^ dS', dK^, dgamma
    // dS' is staged through LDS a quarter of its value rows at a time (QJ rows of [value][key]);
    // the next quarter is loaded into registers while the current one is used.
    {
        constexpr int QJ = DV / 4, QN = QJ * DK / NTH;  // rows and values per thread of a quarter
        float pf[QN];
#pragma unroll
        for (int x = 0; x < QN; ++x) pf[x] = Dg[tid + NTH * x];
        f32x4 dKh[NTK];
#pragma unroll
        for (int x = 0; x < NTK; ++x) dKh[x] = f32x4{0.f, 0.f, 0.f, 0.f};
        float dgam = 0.f;
        for (int qd = 0; qd < 4; ++qd) {
#pragma unroll
            for (int x = 0; x < QN; ++x) {
                const int e = tid + NTH * x;
                sDq[(e / DK) * PK + e % DK] = pf[x];
            }
            __syncthreads();
            if (qd < 3) {
#pragma unroll
                for (int x = 0; x < QN; ++x) pf[x] = Dg[(size_t)(qd + 1) * QJ * DK + tid + NTH * x];
            }
            if (wave < QJ / 16) {  // dUs = K^ dS' for the quarter's value tiles
                const int nt = qd * (QJ / 16) + wave;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mma_big<F32, DK>(acc, [&](int m, int kk) { return Kv(m, kk) * EH(m, kk); },
                                   [&](int kk, int nn) { return sDq[(16 * wave + nn) * PK + kk]; }, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) sdU[(4 * g + i) * PV + 16 * nt + l16] = acc[i];
            }
#pragma unroll
            for (int x = 0; x < NTK; ++x) {  // dK^ += U[:, quarter] dS'[quarter rows]
                const int nt = wave + NW * x;
                if (nt >= NDK) continue;
                dKh[x] = mma_big<F32, QJ>(dKh[x], [&](int m, int kk) { return sU[m * PV + qd * QJ + kk]; },
                                      [&](int kk, int nn) { return sDq[kk * PK + 16 * nt + nn]; }, lane);
            }
            if (tid < DK) {
                for (int jj = 0; jj < QJ; ++jj) dgam += sS[(qd * QJ + jj) * PK + tid] * sDq[jj * PK + tid];
            }
            __syncthreads();
        }
        if (tid < DK) sDg[tid] = dgam;  // dgamma_c
#pragma unroll
        for (int x = 0; x < NTK; ++x) {
            const int nt = wave + NW * x;
            if (nt >= NDK) continue;
            float col = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g + i, c = 16 * nt + l16;
                const float eh = EH(r, c), kh = Kv(r, c) * eh;
                dKa[x][i] += dKh[x][i] * eh;   // dK^ e^{G_last - G}
                dGa[x][i] -= dKh[x][i] * kh;   // - dK^ * K^
                col += dKh[x][i] * kh;
            }
            col += __shfl_xor(col, 16, 64);
            col += __shfl_xor(col, 32, 64);
            if (g == 0) sGl[16 * nt + l16] = col;  // sum over the chunk's rows of dK^ * K^
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- dU = M^T dO + K^ dS', dM
#pragma unroll
    for (int x = 0; x < NTV; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDV) continue;
        f32x4 acc;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = sdU[(4 * g + i) * PV + 16 * nt + l16];
        acc = mma_tile<C>(acc, [&](int m, int kk) { return sM[kk * P16 + m]; },
                          [&](int kk, int nn) { return sdO[kk * PV + 16 * nt + nn]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdU[(4 * g + i) * PV + 16 * nt + l16] = acc[i];
    }
    if (wave == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DV>(acc, [&](int m, int kk) { return sdO[m * PV + kk]; },
                           [&](int kk, int nn) { return sU[nn * PV + kk]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdM[(4 * g + i) * P16 + l16] = (l16 <= 4 * g + i) ? acc[i] : 0.f;
    }
    __syncthreads();

    // ---------------------------------------------------------------- dW = -dU S^T
#pragma unroll
    for (int x = 0; x < NTK; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDK) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DV>(acc, [&](int m, int kk) { return sdU[m * PV + kk]; },
                           [&](int kk, int nn) { return sS[kk * PK + 16 * nt + nn]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sW[(4 * g + i) * PK + 16 * nt + l16] = -acc[i];
    }
    __syncthreads();

    // ---------------------------------------------------------------- dT = dW X^T + dU Y^T
    if (wave == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_big<F32, DK>(acc, [&](int m, int kk) { return sW[m * PK + kk]; },
                           [&](int kk, int nn) { return Xv(nn, kk); }, lane);
        acc = mma_big<F32, DV>(acc, [&](int m, int kk) { return sdU[m * PV + kk]; },
                           [&](int kk, int nn) { return sB[nn] * sV[nn * PV + kk]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdT[(4 * g + i) * P16 + l16] = acc[i];
    }
    __syncthreads();

    // ---------------------------------------------------------------- dX, dY (-> dv, dbeta), dA
    float db[4] = {0.f, 0.f, 0.f, 0.f};  // this wave's part of dbeta for rows 4g+i
#pragma unroll
    for (int x = 0; x < NTK; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDK) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_tile<C>(acc, [&](int m, int kk) { return sT[kk * P16 + m]; },
                          [&](int kk, int nn) { return sW[kk * PK + 16 * nt + nn]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i, c = 16 * nt + l16;
            const float eg = EG(r, c), kt = Kv(r, c) * eg;
            dKa[x][i] += sB[r] * acc[i] * eg;   // b dX e^G
            dGa[x][i] += sB[r] * acc[i] * kt;   // b dX * K~
            db[i] += acc[i] * kt;               // dX * K~
        }
    }
#pragma unroll
    for (int x = 0; x < NTV; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDV) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_tile<C>(acc, [&](int m, int kk) { return sT[kk * P16 + m]; },
                          [&](int kk, int nn) { return sdU[kk * PV + 16 * nt + nn]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i, c = 16 * nt + l16;
            dv[(t0 + r) * DV + c] = sB[r] * acc[i];
            db[i] += acc[i] * sV[r * PV + c];
        }
    }
    if (wave == 3) {  // dA = -strict_tril(T^T dT T^T); dbeta += rowsum(dA * P); dP = diag(b) dA
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = mma_tile<C>(z, [&](int m, int kk) { return sdT[m * P16 + kk]; },
                        [&](int kk, int nn) { return sT[nn * P16 + kk]; }, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) sdA[(4 * g + i) * P16 + l16] = z[i];  // dT T^T
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma_tile<C>(acc, [&](int m, int kk) { return sT[kk * P16 + m]; },
                          [&](int kk, int nn) { return sdA[kk * P16 + nn]; }, lane);
        float dpa[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            dpa[i] = (l16 < r) ? -acc[i] : 0.f;
            db[i] += dpa[i] * sP[r * P16 + l16];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sdT[(4 * g + i) * P16 + l16] = sB[4 * g + i] * dpa[i];  // dP, over dT
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
    __syncthreads();

    // ---------------------------------------------------------------- pairwise terms of M and P
#pragma unroll
    for (int x = 0; x < NTK; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDK) continue;
        const int cn = 16 * nt;
        f32x4 x1 = {0.f, 0.f, 0.f, 0.f}, x2 = x1, x3 = x1, x4 = x1;
        x1 = mma_tile<C>(x1, [&](int m, int kk) { return sdM[m * P16 + kk]; },
                         [&](int kk, int nn) { return Kv(kk, cn + nn) * Em(kk, cn + nn); }, lane);   // dM Km
        x2 = mma_tile<C>(x2, [&](int m, int kk) { return sdM[kk * P16 + m]; },
                         [&](int kk, int nn) { return Qv(kk, cn + nn) * Ep(kk, cn + nn); }, lane);   // dM^T Qp
        x3 = mma_tile<C>(x3, [&](int m, int kk) { return sdT[m * P16 + kk]; },
                         [&](int kk, int nn) { return Kv(kk, cn + nn) * Em(kk, cn + nn); }, lane);   // dP Km
        x4 = mma_tile<C>(x4, [&](int m, int kk) { return sdT[kk * P16 + m]; },
                         [&](int kk, int nn) { return Kv(kk, cn + nn) * Ep(kk, cn + nn); }, lane);   // dP^T Kp
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i, c = cn + l16;
            const float ep = Ep(r, c), em = Em(r, c), qr = Qv(r, c), kr = Kv(r, c);
            const float a1 = x1[i] * ep, a2 = x2[i] * em, a3 = x3[i] * ep, a4 = x4[i] * em;
            dQa[x][i] += a1;
            dKa[x][i] += a2 + a3 + a4;
            dGa[x][i] += qr * a1 - kr * a2 + kr * a3 - kr * a4;
        }
    }

    // ---------------------------------------------------------------- outputs; dg = reverse cumsum of dG
#pragma unroll
    for (int x = 0; x < NTK; ++x) {
        const int nt = wave + NW * x;
        if (nt >= NDK) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i, c = 16 * nt + l16;
            float dg = dGa[x][i];
            if (r == C - 1) dg += sGl[c] + sDg[c] * EG(C - 1, c);  // G_last: K^ and gamma
            dq[(t0 + r) * DK + c] = dQa[x][i];
            dk[(t0 + r) * DK + c] = dKa[x][i];
            sW[r * PK + c] = dg;
        }
    }
    __syncthreads();
    if (tid < DK) {
        float acc = 0.f;
#pragma unroll
        for (int r = C - 1; r >= 0; --r) {
            acc += sW[r * PK + tid];
            da[(t0 + r) * DK + tid] = acc * gpr[r];
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
