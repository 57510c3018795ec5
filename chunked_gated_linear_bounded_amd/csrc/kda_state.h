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
// The slice of S^T stays in the state wave's registers for the whole sequence
// in accumulator layout; by the slot convention of kda_device.h the same
// registers are the B operand of W S^T and the A operand of (S^T)^T Qbar^T, and
// U's accumulators are the B operand of K^^T U -- no shuffles.  All three
// products take fp16 operands: U and S^T are scaled by a power of two from their
// wave-wide maximum magnitude (S^T is kept pre-scaled and rescaled only when
// its maximum leaves [2^11, 2^15); W, Qbar and K^ arrive scaled the same way)
// and the scales are undone exactly on the fp32 results.  Each operand fragment
// is one 16-byte LDS read (tile pairs), and independent output tiles keep
// separate accumulators so consecutive MFMAs do not wait on each other.
//
// Work-group = 3 waves on three SIMDs: wave 0 carries the state (W S^T, U,
// K^^T U, S^T); wave 2 forms the output from the fp16 state operand wave 0
// hands over through LDS (written over W^T in the chunk's own buffer once wave 0
// has read W^T, so the hand-over costs no extra LDS); wave 1 streams chunk
// records into a ring of LDS buffers with direct global->LDS loads (every load
// of a record in flight at once, no staging registers), two chunks ahead.  Two
// barriers per chunk: the first once the state operand is in LDS (the loader
// then refills the buffer of the chunk before), the second when the chunk is
// done.
// Work-group ids are mapped so that all slices of a head land on one XCD and
// share its L2.  The slices of a head read each record in the same order at
// nearly the same time, so one of them takes the HBM miss and the others hit
// in L2; the ring alone then keeps only two records per head in flight, which
// bounds the stage by HBM latency.  The loader therefore also touches its
// slice's share of the record four chunks ahead, so that the ring's loads
// find it in L2.
#pragma once
#include "kda_device.h"
#include "kda_layout.h"

namespace kda {

// VL: each buffer also holds the chunk's 16-byte chunk-table entry after the record.
template <int C, int DK, int DV, bool F32, bool VL = false>
struct StateCfg {
    using E = typename std::conditional<F32, float, __bf16>::type;
    static constexpr int ES = sizeof(E);
    static constexpr KdaLayout L = kda_layout(C, DK, DV, ES);
    static constexpr int ENT = (int)(L.region1 + L.slice);  // VL: the chunk-table entry
    static constexpr int BUF = ENT + (VL ? 16 : 0);
    static constexpr int LDS_MAX = 160 * 1024;
    // direct-load instructions per record (each moves 1 KiB; VL adds the entry's)
    static constexpr int NDMA = (int)((L.region1 + 1023) / 1024 + (L.slice + 1023) / 1024) + (VL ? 1 : 0);
    // three buffers give two chunks of lookahead; the partial wait needs NDMA <= 63
    static constexpr int NBUF = (3 * BUF <= LDS_MAX && NDMA <= 63) ? 3 : (2 * BUF <= LDS_MAX) ? 2 : 1;
    static constexpr int NS = DV / 16;
    // L2 prefetch (three buffers only): each of a head's NS slice work-groups touches its 1/NS
    // share of the record PF chunks ahead, one 4-byte direct load per 128-byte line into a
    // 256-byte sink after the ring, so the ring's own loads find the record in L2
    static constexpr int PF = 4;
    static constexpr int PF_SHARE = (int)(L.stride / NS);
    static constexpr int PF_LINES = (PF_SHARE + 127) / 128, PF_INST = (PF_LINES + 63) / 64;
    static constexpr bool PREFETCH = NBUF == 3 && NDMA + PF_INST <= 63 && NBUF * BUF + 256 <= LDS_MAX;
    static constexpr int SMEM = NBUF * BUF + (PREFETCH ? 256 : 0);
};

// Issue direct global->LDS copies of BYTES (multiple of 16) with one wave:
// each instruction moves 64 x 16 bytes to consecutive LDS addresses.  The
// caller waits for them (vmcnt) before handing the buffer over.
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(lds_u8 *dst, const unsigned char *__restrict__ src, int lane) {
    static_assert(BYTES % 16 == 0, "16-byte units");
    constexpr int UNITS = BYTES / 16, NI = (UNITS + 63) / 64;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int u = i * 64 + lane;
        if (u < UNITS)
            __builtin_amdgcn_global_load_lds(src + (size_t)u * 16, (lds_void *)(dst + i * 1024), 16, 0, 0);
    }
}

// A value every lane holds alike (read from one LDS address), moved to scalar registers.
__device__ __forceinline__ int4 uniform(int4 e) {
    return make_int4(__builtin_amdgcn_readfirstlane(e.x), __builtin_amdgcn_readfirstlane(e.y),
                     __builtin_amdgcn_readfirstlane(e.z), __builtin_amdgcn_readfirstlane(e.w));
}

// Issue the copies of one chunk's record (region 1 + one value slice) and, when `ent` is not
// NULL, of its 16-byte chunk-table entry (one lane) right after them.
template <int R1, int SL>
__device__ __forceinline__ void issue_record(lds_u8 *dst, const unsigned char *__restrict__ rec,
                                             size_t slice_off, int lane, const int4 *ent = nullptr) {
    dma_to_lds<R1>(dst, rec, lane);
    dma_to_lds<SL>(dst + R1, rec + slice_off, lane);
    if (ent != nullptr && lane == 0)
        __builtin_amdgcn_global_load_lds(ent, (lds_void *)(dst + R1 + SL), 16, 0, 0);
}


// VL: packed documents (kda_varlen.h).  Unit hb is then (run p = hb / H of documents, head
// hb % H): it walks the run's chunk records back to back (records head * NCmax + coff[seg[p]]
// ...), each chunk's first token, rows, document and first/last flags taken from the chunk table
// a chunk ahead; at a document's last chunk the state wave stores that document's final state
// and starts the next document from its initial state (loaded a chunk ahead), and only the rows
// that are tokens are stored.  initial_state and final_state are then indexed by (document,
// head), else by unit.
template <int C, int DK, int DV, bool F32, bool VL>
__global__ __launch_bounds__(192, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void kda_state_kernel(
    const unsigned char *__restrict__ ws, typename StateCfg<C, DK, DV, F32, VL>::E *__restrict__ out,
    float *final_state, const float *init_state, int BH, int T, unsigned long long *__restrict__ counts,
    const int4 *__restrict__ ctab, const int *__restrict__ seg, const int *__restrict__ coff, int H, int NCmax,
    float *__restrict__ states, int c0, int NCw)
{
    // states (nullable, fixed-length only): the state each chunk starts from, [BH][NC][DV][DK] float32 in
    // final_state's orientation, for the backward pass; out may then be NULL (no outputs stored).
    // Fixed-length batches: the unit walks chunks c0 .. c0 + NCw - 1 (a window of the sequence)
    // from init_state, whose records the workspace holds as [unit][NCw].
    using Cfg = StateCfg<C, DK, DV, F32, VL>;
    using E = typename Cfg::E;
    using OH = typename std::conditional<F32, float, _Float16>::type;
    using FH = Frag<OH>;
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

    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::SMEM];
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = tid >> 6;
    const int j0 = 16 * slice;
    int NC;                // chunks of this unit
    size_t row0;           // the first token of its head's stream in out (VL) or of its sequence
    const unsigned char *rec0;
    int head = hb, cbase = 0;  // VL: the head, and the run's first chunk in the chunk table
    if constexpr (VL) {
        const int p = hb / H;
        head = hb % H;
        const int d0 = seg[p], d1 = seg[p + 1];
        const int c0 = coff[d0], c1 = coff[d1] < NCmax ? coff[d1] : NCmax;
        NC = c1 > c0 ? c1 - c0 : 0;
        cbase = c0;
        row0 = (size_t)head * T;
        rec0 = ws + ((size_t)head * NCmax + c0) * L.stride;
    } else {  // chunks c0 .. c0 + NCw - 1 of the sequence, records [unit][NCw]
        NC = NCw;
        row0 = (size_t)hb * T + (size_t)c0 * C;
        rec0 = ws + (size_t)hb * NC * L.stride;
    }
    const int4 *ent0 = VL ? ctab + cbase : nullptr;  // VL: the run's chunk-table entries, in chunk order
    // where this lane's part of a state slice is: [document][head][value][key] (VL), [unit][value][key]
    auto state_off = [&](int doc) {
        return ((size_t)(VL ? (size_t)doc * H + head : (size_t)hb) * DV + j0 + l16) * DK + 4 * g;
    };
    const size_t soff = L.region1 + (size_t)slice * L.slice;

    constexpr int NDMA = Cfg::NDMA, PF = Cfg::PF, PF_INST = Cfg::PF_INST;
    // this slice's share of chunk m's record into L2 (m < NC)
    auto prefetch = [&](int m) {
        const unsigned char *src = rec0 + (size_t)m * L.stride + (size_t)slice * Cfg::PF_SHARE;
#pragma unroll
        for (int i = 0; i < PF_INST; ++i) {
            const int line = i * 64 + lane;
            if (line < Cfg::PF_LINES)
                __builtin_amdgcn_global_load_lds(src + (size_t)line * 128, (lds_void *)(lds_base(smem) + NBUF * BUF), 4, 0, 0);
        }
    };
    if (wave == 1 && NC > 0) {
        if constexpr (Cfg::PREFETCH) {  // chunks 2 .. PF - 1 (the loop prefetches chunk n + PF)
            for (int m = 2; m < PF && m < NC; ++m) prefetch(m);
        }
        issue_record<R1B, SLB>(lds_base(smem), rec0, soff, lane, ent0);
        if (NBUF == 3 && NC > 1) {
            issue_record<R1B, SLB>(lds_base(smem) + BUF, rec0 + L.stride, soff, lane, VL ? ent0 + 1 : nullptr);
            wait_vmcnt<NBUF == 3 ? NDMA : 0>();  // chunk 0 has landed
        } else {
            wait_vmcnt<0>();
        }
    }

    // The state slice is kept scaled by 2^sS (wave-uniform), with sS chosen so that its
    // largest magnitude lies in [2^11, 2^15): the fp16 operand is then a plain conversion,
    // and the scale is only adjusted when the maximum leaves that range.
    f32x4 S[NDK];
#pragma unroll
    for (int mt = 0; mt < NDK; ++mt) S[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    int sS = 0;
    // |S 2^sS| < 2^eS (wave-uniform): 15 while the range holds, 14 just after a rescale, ZERO_S
    // while the state is all zero (its product with W then bounds nothing)
    constexpr int ZERO_S = -1000;
    int eS = ZERO_S;
    unsigned int nonfinite = 0;
    // a fresh state taken to the scale the state is kept at (bf16 I/O)
    auto take_scale = [&]() {
        sS = 0;
        eS = ZERO_S;
        if constexpr (!F32) {
            float m = 0.f;
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
            m = wave_max(m);
            if (m != 0.f) eS = 15;  // a non-finite state bounds nothing either way
            if (m > 0.f && __builtin_isfinite(m)) {
                eS = 14;
                sS = pow2_scale(m);
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[mt][i] = ldexp2(S[mt][i], sS);
            }
        }
    };
    if (init_state != nullptr && wave == 0 && (!VL || NC > 0)) {
        // S_0: init_state[..][value j0 + l16][key 16 mt + 4g + i] = S^T[key][value] (read before this
        // work-group writes final_state, which may be the same array)
        const float *ip = init_state + state_off(VL ? ctab[cbase].z : 0);  // the run's first document
#pragma unroll
        for (int mt = 0; mt < NDK; ++mt) S[mt] = *reinterpret_cast<const f32x4 *>(ip + 16 * mt);
        take_scale();
    }
    f32x4 Si[VL ? NDK : 1];  // VL: the next document's initial state, loaded as its predecessor's last chunk starts
#pragma unroll
    for (int mt = 0; mt < (VL ? NDK : 1); ++mt) Si[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Hand-over of the state operand to the output wave: at the start of chunk n the state wave
    // converts S to the fp16 operand once (its own W S^T uses it too) and stores it, with its
    // exponent, over W^T in chunk n's buffer once W^T has been read into registers (LDS
    // accesses of one wave stay in order).  The output wave reads it after the first barrier;
    // the loader refills that buffer only after the chunk's last barrier.  Storing it at the end
    // of chunk n - 1 instead puts the stores in front of that chunk's last barrier and converts
    // S twice.
    auto hand_over = [&](int buf, const FH (&sh)[NKB], int e) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            st_frag_lds(lds_base(smem) + buf * BUF + L.wt + kb * 512 * (int)sizeof(OH), lane, sh[kb]);
        if (lane == 0) reinterpret_cast<int *>(smem + buf * BUF + L.scl)[3] = e;
    };
    auto state_operand = [&](FH (&sh)[NKB]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = S[2 * kb + j / 4][j % 4];
            sh[kb] = FH::make(x);
        }
    };
    barrier_lds();  // chunk 0 has landed

    for (int n = 0; n < NC; ++n) {
        unsigned char *cur = smem + (n % NBUF) * BUF;
        const OH *bWT = reinterpret_cast<const OH *>(cur + L.wt);
        const OH *bQB = reinterpret_cast<const OH *>(cur + L.qbt);
        const OH *bKH = reinterpret_cast<const OH *>(cur + L.kh);
        const float *bG = reinterpret_cast<const float *>(cur + L.gam);
        int *bScl = reinterpret_cast<int *>(cur + L.scl);
        const OH *bU = reinterpret_cast<const OH *>(cur + L.region1 + L.ut);
        const OH *bO = reinterpret_cast<const OH *>(cur + L.region1 + L.oit);
        const int *bSS = reinterpret_cast<const int *>(cur + L.region1 + L.ssc);
        constexpr int PE = 2 * TE;  // elements per stored tile pair

        const OH *shx = reinterpret_cast<const OH *>(cur + L.wt);  // chunk n's state operand
        const int *shs = reinterpret_cast<const int *>(cur + L.scl) + 3;

        // ---- W^T into the state wave's registers, then the state operand over it
        FH wt[NKB][NT], So[NKB], Sh[NKB];
        f32x4 ut[NT];
        int eW = 0, eK = 0, eU = 0, sSo = 0;
        if (wave == 0) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) wt[kb][tt] = FH::load_pair(bWT + (kb * NT + tt) * PE, lane);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) ut[tt] = ld_tile(bU + tt * TE, lane);
            eW = bScl[0];
            eK = bScl[2];
            eU = bSS[0];
            state_operand(Sh);
            hand_over(n % NBUF, Sh, sS);
        }
        barrier_lds();  // the state operand is in LDS

        if (wave == 1) {
            // ---- loader: the record two chunks ahead
            if (NBUF == 3) {
                if (n + 2 < NC) {
                    issue_record<R1B, SLB>(lds_base(smem) + ((n + 2) % 3) * BUF, rec0 + (size_t)(n + 2) * L.stride, soff,
                                           lane, VL ? ent0 + n + 2 : nullptr);
                    if (Cfg::PREFETCH && n + PF < NC) {
                        prefetch(n + PF);
                        wait_vmcnt<Cfg::PREFETCH ? NDMA + PF_INST : 0>();  // chunk n + 1 has landed
                    } else {
                        wait_vmcnt<NBUF == 3 ? NDMA : 0>();  // chunk n + 1 has landed
                    }
                } else {
                    wait_vmcnt<0>();
                }
            } else if (NBUF == 2 && n + 1 < NC) {
                issue_record<R1B, SLB>(lds_base(smem) + ((n + 1) & 1) * BUF, rec0 + (size_t)(n + 1) * L.stride, soff,
                                       lane, VL ? ent0 + n + 1 : nullptr);
                wait_vmcnt<0>();
            }
        } else if (wave == 0) {
            // ---- state wave: U = U~ - W S^T;  S^T <- diag(gamma) S^T + K^^T U
            int4 e_cur = make_int4(0, 0, 0, 0);
            if constexpr (VL) {  // this chunk's entry; at a document's last chunk, the next one's initial state
                e_cur = uniform(*reinterpret_cast<const int4 *>(cur + Cfg::ENT));
                const int next_doc = (e_cur.w >> 2) - 1;
                if (init_state != nullptr && (e_cur.w & 2) && next_doc >= 0) {
                    const float *ip = init_state + state_off(next_doc);
#pragma unroll
                    for (int mt = 0; mt < NDK; ++mt) Si[mt] = *reinterpret_cast<const f32x4 *>(ip + 16 * mt);
                }
            }
            if (states != nullptr) {  // the state chunk n starts from, unscaled
                float *sp = states + (((size_t)hb * NC + n) * DV + j0 + l16) * DK + 4 * g;
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt) {
                    f32x4 x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] = ldexp2(S[mt][i], -sS);
                    *reinterpret_cast<f32x4 *>(sp + 16 * mt) = x;
                }
            }
            f32x4 P[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) P[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) P[tt] = mma(wt[kb][tt], Sh[kb], P[tt]);
            FH kh[NTKB][NDK];  // read while W S^T is in flight
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb)
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt) kh[kb][mt] = FH::load_pair(bKH + (kb * NDK + mt) * PE, lane);
            f32x4 gm[NDK];
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) gm[mt] = *reinterpret_cast<const f32x4 *>(bG + 16 * mt + 4 * g);
            // U = U~ - W S^T (both scalings are exact, the difference rounds once), formed at the
            // working scale 2^sW: the state's own scale unless U~ is far larger than the state (one
            // that has decayed to almost nothing), when the state is taken down to U~'s.  Every
            // factor is then a moderate power of two, whatever the state has decayed by.
            const int sW = min(sS, eU + 16);
            const float fW = ldexp2(1.f, sW - sS - eW), fU = ldexp2(1.f, sW - eU);
            f32x4 U[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) U[tt][i] = fmaf(ut[tt][i], fU, -(P[tt][i] * fW));
            // U's fp16 scale from bounds rather than from its wave-wide maximum (a chain of
            // cross-lane steps on the state's critical path): the stored U~ and W^T blocks are below
            // 2^14 and the state operand below 2^eS, so
            //   |U| < 2^(14 + sW - eU) + 2^(14 + eS + log2 DK + sW - sS - eW)
            // (no second term while the state is zero) and U 2^sU stays below 2^15.  A loose bound only moves U's smallest elements nearer
            // fp16's subnormals, far below the rounding of its largest ones.
            constexpr int LOG2DK = DK == 128 ? 7 : 6;
            static_assert(DK == 64 || DK == 128, "dk of 64 or 128");
            const int sU = F32 ? 0 : 14 - max(14 + sW - eU, eS == ZERO_S ? ZERO_S : 14 + eS + LOG2DK + sW - sS - eW);
            FH Uh[NTKB];
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 2 * kb + j / 4;
                    x[j] = (t < NT) ? ldexp2(U[t < NT ? t : 0][j % 4], sU) : 0.f;
                }
                Uh[kb] = FH::make(x);
            }
            // independent accumulators per 16-row dk tile
            f32x4 A[NDK];
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) A[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb)
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt) A[mt] = mma(kh[kb][mt], Uh[kb], A[mt]);
            if (sW != sS) {  // rare
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[mt][i] = ldexp2(S[mt][i], sW - sS);
                sS = sW;
            }
            const float unS = ldexp2(1.f, -(sU + eK));
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[mt][i] = fmaf(A[mt][i], unS, S[mt][i] * gm[mt][i]);
            if constexpr (!F32) {  // keep the scaled maximum in [2^11, 2^15)
                float m = 0.f;
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[mt][i]));
                if (!wave_max_in(m, 2048.f, 32768.f)) {  // the wave-wide maximum only when it is needed
                    m = wave_max(m);
                    eS = m == 0.f ? ZERO_S : 15;
                    if (m > 0.f && __builtin_isfinite(m) && (m >= 32768.f || m < 2048.f)) {
                        const int d = pow2_scale(m);
#pragma unroll
                        for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) S[mt][i] = ldexp2(S[mt][i], d);
                        sS += d;
                        eS = 14;
                    }
                } else {
                    eS = 15;
                }
            }
            if constexpr (VL) {
                if (e_cur.w & 2) {  // the last chunk of its document
                    if (final_state != nullptr) {
                        float *fp = final_state + state_off(e_cur.z);
#pragma unroll
                        for (int mt = 0; mt < NDK; ++mt) {
                            f32x4 x;
#pragma unroll
                            for (int i = 0; i < 4; ++i) x[i] = ldexp2(S[mt][i], -sS);
                            *reinterpret_cast<f32x4 *>(fp + 16 * mt) = x;
                        }
                    }
                    if (n + 1 < NC) {  // the next document starts from its own state
#pragma unroll
                        for (int mt = 0; mt < NDK; ++mt) S[mt] = init_state != nullptr ? Si[mt] : f32x4{0.f, 0.f, 0.f, 0.f};
                        take_scale();
                    }
                }
            }
        } else {
            // ---- output wave: O^T = Oi^T + (S^T)^T Qbar^T with the state the chunk started from
            const int4 e_cur = VL ? uniform(*reinterpret_cast<const int4 *>(cur + Cfg::ENT)) : make_int4(0, 0, 0, 0);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) So[kb] = FH::load_pair(shx + kb * 512, lane);
            sSo = *shs;
            FH qb[NKB][NT];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) qb[kb][tt] = FH::load_pair(bQB + (kb * NT + tt) * PE, lane);
            f32x4 oi[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) oi[tt] = ld_tile(bO + tt * TE, lane);
            const float unO = ldexp2(1.f, -(sSo + bScl[1])), unI = ldexp2(1.f, -bSS[1]);
            f32x4 O[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) O[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) O[tt] = mma(So[kb], qb[kb][tt], O[tt]);
            const size_t trow = VL ? row0 + (size_t)e_cur.x : row0 + (size_t)n * C;
            const int nval = VL ? e_cur.y : C;  // rows of this chunk that are tokens
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 o;
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = fmaf(O[tt][i], unO, oi[tt][i] * unI);
                if ((VL && 16 * tt + l16 >= nval) || out == nullptr) continue;
                // lane holds out[token 16 tt + l16][value j0 + 4g + i]
                E *op = out + (trow + 16 * tt + l16) * DV + j0 + 4 * g;
                if constexpr (F32) {
                    *reinterpret_cast<f32x4 *>(op) = o;
                } else {
                    bf16x4 bo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) bo[i] = (__bf16)o[i];
                    *reinterpret_cast<bf16x4 *>(op) = bo;
                    // what was stored, for the optional non-finite count
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = (float)bo[i];
                }
                if (counts != nullptr) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) nonfinite += !__builtin_isfinite(o[i]);
                }
            }
        }
        barrier_lds();
        if (NBUF == 1) {
            if (wave == 1 && n + 1 < NC) {
                issue_record<R1B, SLB>(lds_base(smem), rec0 + (size_t)(n + 1) * L.stride, soff, lane,
                                       VL ? ent0 + n + 1 : nullptr);
                wait_vmcnt<0>();
            }
            barrier_lds();
        }
    }
    if (!VL && wave == 0 && final_state != nullptr) {
        // final_state[hb][value j0 + l16][key 16 mt + 4g + i] = S^T[key][value]
        float *fp = final_state + ((size_t)hb * DV + j0 + l16) * DK + 4 * g;
#pragma unroll
        for (int mt = 0; mt < NDK; ++mt) {
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = ldexp2(S[mt][i], -sS);
            *reinterpret_cast<f32x4 *>(fp + 16 * mt) = x;
        }
    }
    if (wave == 2 && counts != nullptr && nonfinite) atomicAdd(&counts[1], (unsigned long long)nonfinite);
}

}  // namespace kda
