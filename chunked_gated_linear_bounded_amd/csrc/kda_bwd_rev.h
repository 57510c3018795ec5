// Reverse pass of the backward for bf16 inputs: carries dS', the gradient of the state a 16-token
// chunk ends in, from the last chunk to the first for one head and one 16-wide value slice,
//   dS = diag(gamma) dS' + Qbar^T dO - W^T (K^ dS'),
// storing dS' for every chunk and giving dL/dS_0 at the end (the chunk form written out at the
// top of kda_bwd.h; "Breaking Through Trillion-Parameter Multimodal MoE ...", sec. 2.1).
//
// The chain is a few short products per chunk, so its length is set by latency:
//   - every product is a 16x16x16 bf16 MFMA whose B operand is an accumulator tile as it stands
//     (lane group g holds rows 4 g .. 4 g + 3 of its column, which is the B layout of that MFMA):
//     K^ dS' takes the wave's dS' tiles, W^T P takes P;
//   - dS' and P, fp32, are split into bf16 hi + lo (about 16 significand bits, the full range);
//     the record's fp16 blocks are exact as hi + lo, and their power-of-two scales are applied to
//     the products;
//   - one wave per 16-row key tile of the slice (eight at dk = 128, two per SIMD) forms its part of
//     K^ dS' over its tile, and one barrier per chunk hands the parts to everyone;
//   - each chunk's operands are read from the ring and split during the previous chunk's update,
//     and Qbar^T dO, which does not depend on dS', before the barrier.
// One more wave streams each chunk's record and dout block into a ring of LDS slots (four where they
// fit) with direct global->LDS loads, as many chunks ahead as the ring holds, touches the lines
// of a chunk eight ahead into L2 (each slice a share of them) so that the ring's loads hit there,
// and alone waits on its memory counter.
#pragma once
#include "kda_bwd.h"

namespace kda {

template <int DK, int DV>
__global__ __launch_bounds__((DK / 16 + 1) * 64) void kda_bwd_rev_kernel(
    const unsigned char *__restrict__ ws, const __bf16 *__restrict__ dout, const float *__restrict__ dfinal, int T,
    int BH, float *__restrict__ dstates, float *__restrict__ dinit)
{
    constexpr KdaLayout L = kda_layout(16, DK, DV, 2);
    constexpr int NS = DV / 16, NDK = DK / 16, NCW = NDK, NTW = 1;  // one compute wave per key tile
    static_assert(NDK == 4 || NDK == 8, "dk of 64 or 128");
    constexpr int R1 = (int)L.region1, NU = (R1 + 15) / 16;  // 16-byte units of region 1
    constexpr int NBLK = (NU + 63) / 64;                     // 1 KiB direct-load blocks
    constexpr int RB = NBLK * 1024, SLOT = RB + 1024;        // record + dout block
    constexpr int NDMA = NBLK + 1;                           // loader instructions per chunk
    // ring depth: four slots where they fit in 80 KB (the loader keeps NSLOT - 2 chunks in flight
    // beyond the one it waits for); the work-group then leaves room in LDS for one of the state
    // recompute (about 62 KB), which runs at the same time on another stream
    constexpr int NSLOT = (4 * SLOT <= 80 * 1024 && 1 + 2 * (NDMA + 1) <= 63) ? 4 : 3;
    // vmem instructions the loader issues after a chunk's ring loads before it waits for that
    // chunk: its L2 touch in the same iteration, then a ring chunk and a touch per iteration
    constexpr int AFTER = 1 + (NSLOT - 2) * (NDMA + 1);
    static_assert(AFTER <= 63, "partial wait needs the count in the vmcnt field");
    // L2 touch: PF chunks ahead each slice work-group loads 4 bytes of every 128-byte line of its
    // share of region 1 and of its own dout rows, so the ring's loads find them in L2
    constexpr int PF = 8, R1L = (R1 + 127) / 128, SHL = (R1L + NS - 1) / NS;
    static_assert(PF > NSLOT - 1 && SHL + 16 <= 64, "one touch instruction per chunk");

    __shared__ __attribute__((aligned(1024))) unsigned char sRing[NSLOT * SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char sSink[256];
    __shared__ f32x4 sPp[2][NCW][64];  // each compute wave's part of K^ dS', as its lanes hold it; two sets

    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave <= NCW);  // the range readfirstlane hides
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
        // dout block: 16 rows x 16 values of this slice, 16 bytes per lane (two lanes per row)
        const int row = min(lane >> 1, 15), part = lane & 1;
        const unsigned char *srow = reinterpret_cast<const unsigned char *>(
            dout + ((size_t)bh * T + (size_t)n * 16 + row) * DV + j0);
        __builtin_amdgcn_global_load_lds(srow + 16 * part, (lds_void *)(dst + RB), 16, 0, 0);
    };

    auto touch = [&](int m) {
        const int line = slice * SHL + lane, row = min(max(lane - SHL, 0), 15);
        const unsigned char *src = lane < SHL && line < R1L
            ? rec0 + (size_t)m * L.stride + (size_t)line * 128
            : reinterpret_cast<const unsigned char *>(dout + ((size_t)bh * T + (size_t)m * 16 + row) * DV + j0);
        __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base(sSink), 4, 0, 0);
    };
    // the loader, in the iteration of chunk n, issues chunk n - (NSLOT - 1) into the ring and
    // touches chunk n - PF, then waits until chunk n - 1 has landed; AFTER instructions were issued
    // after that chunk's once every one of them was (n >= PF), else it waits for all
    auto wait_next = [&](int n) {
        if (n < 1) return;
        if (n >= PF) wait_vmcnt<AFTER>();
        else wait_vmcnt<0>();
    };

    // dS' of the last chunk: dfinal (or zero); wave w's tile is key rows 16 w .. 16 w + 15,
    // held as an accumulator (lane (g, j) holds rows 4 g + i of value column j)
    f32x4 D[NTW];
#pragma unroll
    for (int x = 0; x < NTW; ++x) {
        const int mt = wave + NCW * x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 16 * mt + 4 * g + i;
            D[x][i] = (wave < NCW && dfinal != nullptr) ? dfinal[((size_t)bh * DV + j0 + l16) * DK + c] : 0.f;
        }
    }
    // A chunk's operands, read from its ring slot and split one chunk ahead, off the chain:
    // K^[r][16 mt + 4 g + i] (A of K^ dS'), W^T and Qbar^T [16 mt + r][4 g + i] (A of the update),
    // as stored (their power-of-two scales fK, -fW, fQ are applied to the products), gamma of the
    // wave's key rows, the dout block as the B operand of Qbar^T dO.
    // The record keeps four consecutive rows of a column together (the operand order of the
    // forward's products), and these operands need four consecutive columns of a row, so each is
    // one transpose read: lane (g, s) addresses the 8 bytes of the stored run that lane
    // (g, 4 (s & 3) + r) needs in slot s >> 2 (r = 0..3).  Four 2-byte reads per operand instead
    // met every bank four times over.
    struct Ops {
        bf16x4 kh[NTW], kl[NTW], wh[NTW], wl[NTW], qh[NTW], ql[NTW], ob;
        f32x4 gm[NTW];
        float fK, fW, fQ;
    };
    auto prefetch = [&](int s) {
        Ops o;
        const unsigned char *cur = sRing + s * SLOT;
        const lds_u8 *curl = lds_base(sRing) + s * SLOT;
        const float *rG = reinterpret_cast<const float *>(cur + L.gam);
        const int *rS = reinterpret_cast<const int *>(cur + L.scl);
        o.fW = -ldexp2(1.f, -rS[0]);
        o.fQ = ldexp2(1.f, -rS[1]);
        o.fK = ldexp2(1.f, -rS[2]);
        const int p = l16 & 3, kk = l16 >> 2;  // this lane addresses run 16 p + 4 g + kk of a tile
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int mt = wave + NCW * x;
            // K^ [token][key]: key tile mt, tile rows 0..15 (C = 16: the first tile of its pair);
            // W^T, Qbar^T [key][token]: key tile mt, half mt & 1 of pair mt / 2
            const f16x4 kr = ld_tr16<f16x4>(curl + L.kh + 16 * (mt * 64 + 16 * p + 4 * g + kk));
            const int wo = 16 * ((mt >> 1) * 64 + 16 * p + 4 * g + kk) + 8 * (mt & 1);
            const f16x4 wr = ld_tr16<f16x4>(curl + L.wt + wo);
            const f16x4 qr = ld_tr16<f16x4>(curl + L.qbt + wo);
            float ka[4], wa[4], qa[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ka[i] = (float)kr[i];
                wa[i] = (float)wr[i];
                qa[i] = (float)qr[i];
            }
            split4(ka, o.kh[x], o.kl[x]);
            split4(wa, o.wh[x], o.wl[x]);
            split4(qa, o.qh[x], o.ql[x]);
            o.gm[x] = *reinterpret_cast<const f32x4 *>(rG + 16 * mt + 4 * g);
        }
        // dout block [token][16 values]: rows 4 g .. 4 g + 3 of column l16
        o.ob = ld_tr16<bf16x4>(curl + RB + 2 * (16 * (4 * g + kk) + 4 * p));
        return o;
    };

    if (wave == NCW) {  // chunks NC-1 .. NC-NSLOT+1 into the ring, the chunks after them touched
#pragma unroll
        for (int s = 0; s < NSLOT - 1; ++s)
            if (NC - 1 - s >= 0) issue(NC - 1 - s, s);
        for (int s = NSLOT - 1; s < PF && NC - 1 - s >= 0; ++s) touch(NC - 1 - s);
        wait_vmcnt<0>();
    }
    barrier_lds();  // chunk NC-1 has landed
    Ops op;
    if (wave < NCW && NC > 0) op = prefetch(0);

    // One barrier per chunk: it publishes the parts of P (two alternating sets, so a wave
    // that runs ahead never overwrites a set another wave still reads) and chunk n - 1's slot;
    // the loader refills the slot of chunk n + 1, whose operands were read two barriers before.
    for (int it = 0; it < NC; ++it) {
        const int n = NC - 1 - it, ps = it & 1;
        f32x4 qdo[NTW];
        if (wave == NCW) {
            if (n - (NSLOT - 1) >= 0) issue(n - (NSLOT - 1), (it + NSLOT - 1) % NSLOT);
            if (n - PF >= 0) touch(n - PF);
            wait_next(n);  // chunk n - 1 has landed (the ones after it may be in flight)
        } else {
            // this wave's part of P = K^ dS' (16 x 16): A = K^[:, key tile], B = the dS' tile
            f32x4 pt[NTW];
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                bf16x4 dh, dl;
                split4(D[x], dh, dl);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(op.kh[x], dh, acc);
                acc = mfma16(op.kl[x], dh, acc);
                pt[x] = mfma16(op.kh[x], dl, acc);
            }
            f32x4 pp = pt[0];
#pragma unroll
            for (int x = 1; x < NTW; ++x) pp += pt[x];
            sPp[ps][wave][lane] = pp * op.fK;
            // dS' of this chunk's end, for the chunk-parallel stage: dstates[bh][n][value][key]
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                const int mt = wave + NCW * x;
                *reinterpret_cast<f32x4 *>(dstates + (((size_t)bh * NC + n) * DV + j0 + l16) * DK + 16 * mt + 4 * g) = D[x];
            }
            // diag(gamma) dS' + Qbar^T dO: the part of the update that does not wait for P
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(op.qh[x], op.ob, acc);
                acc = mfma16(op.ql[x], op.ob, acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) qdo[x][i] = op.gm[x][i] * D[x][i] + op.fQ * acc[i];
            }
        }
        barrier_lds();  // the four parts of P are in; chunk n - 1 has landed
        if (wave < NCW) {
            f32x4 pw[NCW];
#pragma unroll
            for (int w = 0; w < NCW; ++w) pw[w] = sPp[ps][w][lane];
            const Ops cur = op;
            if (n >= 1) op = prefetch((it + 1) % NSLOT);  // chunk n - 1's operands, read during the update
#pragma unroll
            for (int h = NCW / 2; h >= 1; h /= 2)
#pragma unroll
                for (int w = 0; w < h; ++w) pw[w] += pw[w + h];
            float pv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) pv[i] = pw[0][i];
            bf16x4 ph, pl;
            split4(pv, ph, pl);
            // dS = diag(gamma) dS' + Qbar^T dO - W^T P  (rows of this wave's key tiles)
#pragma unroll
            for (int x = 0; x < NTW; ++x) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma16(cur.wh[x], ph, acc);
                acc = mfma16(cur.wl[x], ph, acc);
                acc = mfma16(cur.wh[x], pl, acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) D[x][i] = qdo[x][i] + cur.fW * acc[i];
            }
        }
    }
    if (dinit != nullptr && wave < NCW) {
#pragma unroll
        for (int x = 0; x < NTW; ++x) {
            const int mt = wave + NCW * x;
            *reinterpret_cast<f32x4 *>(dinit + ((size_t)bh * DV + j0 + l16) * DK + 16 * mt + 4 * g) = D[x];
        }
    }
}

}  // namespace kda
