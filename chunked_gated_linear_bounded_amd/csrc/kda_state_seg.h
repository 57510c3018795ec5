// Sequential stage with the sequence cut into segments (one GPU, many work-groups per head).
//
// The state of a head is carried chunk to chunk ("Trillion-Parameter MoE Multimodal Models:
// Engineering Long-Context ...", sec. 3.2):
//   U = U~ - W S^T,   O = Oi + Qbar S^T,   S^T <- diag(gamma) S^T + K^^T U,
// so each chunk is the affine map S^T <- A_c S^T + B_c with A_c = diag(gamma) - K^^T W.  A
// segment of chunks therefore maps its incoming state X to Phi X + S_loc, where Phi is the
// product of its A_c and S_loc the state it ends in from zero -- the same decomposition that
// lets context-parallel ranks each take a piece of the sequence ("Breaking Through
// Trillion-Parameter Multimodal MoE ...", sec. 3), used here inside one GPU so that a head with
// thousands of chunks is walked by many work-groups at once:
//   pass 0 (kda_seg_state_kernel<.., 0>): per (head, segment) but the last, the end state from
//     zero (the first segment: from the true initial state) and, for segments after the first,
//     Phi, formed by running the identity's columns through the same chain with U~ = 0;
//   kda_seg_scan_kernel: X_{j+1} = Phi_j X_j + S_loc_j in fp32, segment by segment;
//   pass 1 (kda_seg_state_kernel<.., 1>): per (head, segment), the chain again from X_j, with the
//     outputs; the last segment writes final_state.
//
// A work-group carries every value slice of its (head, segment): four waves, one per SIMD, each
// with NCH independent chains (16-column slices of S^T, or of Phi in pass 0) whose products share
// the operand fragments the wave reads from LDS.  The part of each chunk's record every chain
// reads (W^T, K^, gamma and the exponents; pass 1 also Qbar^T) streams into a ring of LDS slots
// with direct global->LDS loads, each of the NW waves issuing every NW-th 1 KiB load and waiting for its
// own with a partial vmcnt (vector-memory loads of a wave return in order), so that the ring
// runs depth - 1 chunks ahead.  The per-slice blocks (U~, Oi^T and their exponents) are read by
// the chain that owns them straight into registers, a chunk ahead.  Operand formats, scalings
// and the range discipline of the state are those of kda_state.h: fp16 operands block-scaled by
// powers of two, the state kept pre-scaled with its maximum in [2^11, 2^15).
#pragma once
#include "kda_device.h"
#include "kda_layout.h"

namespace kda {

template <int C, int DK, int DV, bool F32, int PASS>
struct SegCfg {
    using E = typename std::conditional<F32, float, __bf16>::type;
    using OH = typename std::conditional<F32, float, _Float16>::type;
    static constexpr int ES = sizeof(E);
    static constexpr KdaLayout L = kda_layout(C, DK, DV, ES);
    static constexpr KdaSegRing R = kda_seg_ring(L, PASS);
    static constexpr int NT = C / 16, NDK = DK / 16, NDV = DV / 16, NKB = DK / 32, NTKB = (NT + 1) / 2;
    static constexpr int NCHAIN = PASS ? NDV : NDV + NDK;  // pass 0: state slices, then Phi slices
    // eight waves (two per SIMD, so that one's waits are hidden by the other's work) where the
    // chains divide evenly, else four.  Pass 0 with 16-bit records and sixteen chains (dk = dv =
    // 128) takes sixteen waves, one chain each: four per SIMD within 128 registers, so that the
    // chains' MFMA and LDS latencies overlap further (each wave then reads its own fragments)
    static constexpr int NW = (PASS == 0 && !F32 && NCHAIN == 16) ? 16 : (NCHAIN % 8 == 0 ? 8 : 4);
    static constexpr int NCH = NCHAIN / NW;
    static constexpr int THREADS = NW * 64;
    static_assert(NCHAIN % NW == 0, "chains per wave");
    // offsets inside a ring slot
    static constexpr int S_WT = 0;
    static constexpr int S_QB = (int)L.qbt;  // pass 1 only
    static constexpr int S_KH = PASS ? (int)L.kh : R.p1_len;
    static constexpr int S_GAM = S_KH + (int)(L.gam - L.kh);
    static constexpr int S_SCL = S_KH + (int)(L.scl - L.kh);
    static constexpr int NI1 = (R.p1_len + 1023) / 1024, NI = R.ndma;
    static constexpr int CNT_HI = (NI + NW - 1) / NW, CNT_LO = NI / NW, NHI = NI % NW;
    static constexpr int NR = R.depth;
    static constexpr int SMEM = NR * R.slot;
    static constexpr bool OK = kda_seg_ring_ok(R);
};

// A chain's per-chunk slice blocks, read into registers a chunk ahead: U~ (and, pass 1, Oi^T)
// as this lane's 4 values of each token tile, and their exponents.
template <bool F32, int NT, bool OUT>
struct SliceRegs {
    using V4 = typename std::conditional<F32, f32x4, f16x4>::type;
    V4 u[NT];
    V4 o[OUT ? NT : 1];
    int eu, eo;
};

template <int C, int DK, int DV, bool F32, int PASS>
__global__ __launch_bounds__((SegCfg<C, DK, DV, F32, PASS>::THREADS), 1) void kda_seg_state_kernel(
    const unsigned char *__restrict__ ws, typename SegCfg<C, DK, DV, F32, PASS>::E *__restrict__ out,
    float *final_state, const float *init_state, float *__restrict__ segbuf, float *__restrict__ phibuf, int U,
    int NC, int nseg, int seglen, int T, unsigned long long *__restrict__ counts)
{
    // Grid: pass 0 U * (nseg - 1) work-groups, pass 1 U * nseg; id = segment * U + unit.
    // init_state may be final_state: with several segments pass 0 copies it to the last slot of
    // segbuf and pass 1 reads that copy; with one, each chain reads its slice before it writes it.
    using Cfg = SegCfg<C, DK, DV, F32, PASS>;
    using E = typename Cfg::E;
    using OH = typename Cfg::OH;
    using FH = Frag<OH>;
    using SR = SliceRegs<F32, Cfg::NT, PASS == 1>;
    using V4 = typename SR::V4;
    constexpr KdaLayout L = Cfg::L;
    constexpr KdaSegRing R = Cfg::R;
    constexpr int NT = Cfg::NT, NDK = Cfg::NDK, NDV = Cfg::NDV, NKB = Cfg::NKB, NTKB = Cfg::NTKB;
    constexpr int NW = Cfg::NW, NCH = Cfg::NCH, NR = Cfg::NR, SLOT = R.slot;
    constexpr int TE = 256, PE = 2 * TE;
    static_assert(Cfg::OK, "ring does not fit");

    __shared__ __attribute__((aligned(1024))) unsigned char smem[Cfg::SMEM];

    const int id = blockIdx.x;
    const int unit = id % U, seg = id / U;
    const int cb = seg * seglen;
    const int NCs = NC - cb < seglen ? NC - cb : seglen;  // >= 1: segments are never empty
    const unsigned char *rec0 = ws + ((size_t)unit * NC + cb) * L.stride;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    __builtin_assume(wave >= 0 && wave < NW);
    const bool hi = wave < Cfg::NHI || Cfg::NHI == 0;  // issues CNT_HI loads per chunk (else CNT_LO)

    // this wave's share of chunk m's ring part into slot m % NR
    auto issue = [&](int m) {
        const unsigned char *src = rec0 + (size_t)m * L.stride;
        lds_u8 *dst = lds_base(smem) + (m % NR) * SLOT;
#pragma unroll
        for (int j = 0; j < Cfg::CNT_HI; ++j) {
            const int i = wave + NW * j;
            if (i >= Cfg::NI) break;
            if (i < Cfg::NI1) {
                const int u = i * 64 + lane;
                if (u < R.p1_len / 16)
                    __builtin_amdgcn_global_load_lds(src + R.p1_src + (size_t)u * 16, (lds_void *)(dst + i * 1024), 16, 0, 0);
            } else {
                const int ii = i - Cfg::NI1;
                const int u = ii * 64 + lane;
                if (u < R.p2_len / 16)
                    __builtin_amdgcn_global_load_lds(src + R.p2_src + (size_t)u * 16,
                                                     (lds_void *)(dst + R.p1_len + ii * 1024), 16, 0, 0);
            }
        }
    };

    // chain c of this wave: index gi = wave + NW c; gi < NDV: state slice gi (columns 16 gi of
    // S^T), else (pass 0) Phi slice gi - NDV (columns 16 (gi - NDV) of Phi)
    // (a compile-time property of c when NDV is a multiple of NW).  The first segment's Phi is
    // not needed; its chains run anyway, so that no product sits behind a branch.
    auto is_phi = [&](int c) { return NDV % NW == 0 ? NW * c >= NDV : wave + NW * c >= NDV; };
    auto col0 = [&](int c) { return 16 * (is_phi(c) ? wave + NW * c - NDV : wave + NW * c); };

    auto load_slice = [&](SR &r, int c, int m) {
        if (is_phi(c)) return;
        const unsigned char *sl = rec0 + (size_t)m * L.stride + L.region1 + (size_t)(col0(c) / 16) * L.slice;
        const int *e = reinterpret_cast<const int *>(sl + L.ssc);
        r.eu = e[0];
        r.eo = e[1];
        const OH *ut = reinterpret_cast<const OH *>(sl + L.ut);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) r.u[tt] = *reinterpret_cast<const V4 *>(ut + tt * TE + lane * 4);
        if constexpr (PASS == 1) {
            const OH *oi = reinterpret_cast<const OH *>(sl + L.oit);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) r.o[tt] = *reinterpret_cast<const V4 *>(oi + tt * TE + lane * 4);
        }
    };

    // ---- the chains' states, kept scaled by 2^sS with the maximum in [2^11, 2^15) (bf16 I/O)
    f32x4 S[NCH][NDK];
    int sS[NCH];
    // |S 2^sS| < 2^eS per chain (wave-uniform): 15 while the range holds, 14 just after a
    // rescale, ZERO_S while the chain's state is all zero
    constexpr int ZERO_S = -1000;
    int eS[NCH];
    auto take_scale = [&](int c) {
        sS[c] = 0;
        eS[c] = ZERO_S;
        if constexpr (!F32) {
            float m = 0.f;
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[c][mt][i]));
            m = wave_max(m);
            if (m != 0.f) eS[c] = 15;  // a non-finite state bounds nothing either way
            if (m > 0.f && __builtin_isfinite(m)) {
                eS[c] = 14;
                sS[c] = pow2_scale(m);
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[c][mt][i] = ldexp2(S[c][mt][i], sS[c]);
            }
        }
    };
    // this lane's part of a [cols][DK] fp32 block at column col (l16) and keys 16 mt + 4 g + i
    auto lane_off = [&](int col) { return (size_t)(col + l16) * DK + 4 * g; };
    const size_t sstride = (size_t)DV * DK, pstride = (size_t)DK * DK;
    float *segu = segbuf + (size_t)unit * nseg * sstride;  // this unit's segment states
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const float *src = nullptr;  // NULL: zero
        if (!is_phi(c)) {
            if (PASS == 0)
                src = seg == 0 ? init_state : nullptr;
            else if (seg > 0)
                src = segu + (size_t)(seg - 1) * sstride;
            else
                src = nseg > 1 ? (init_state != nullptr ? segu + (size_t)(nseg - 1) * sstride : nullptr) : init_state;
            if (src == init_state && init_state != nullptr) src = init_state + (size_t)unit * sstride;
        }
        const size_t off = lane_off(col0(c));
#pragma unroll
        for (int mt = 0; mt < NDK; ++mt) {
            if (src != nullptr) {
                S[c][mt] = *reinterpret_cast<const f32x4 *>(src + off + 16 * mt);
            } else if (is_phi(c)) {  // the identity's columns
#pragma unroll
                for (int i = 0; i < 4; ++i) S[c][mt][i] = (16 * mt + 4 * g + i == col0(c) + l16) ? 1.f : 0.f;
            } else {
                S[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        if (PASS == 0 && seg == 0 && nseg > 1 && init_state != nullptr && !is_phi(c)) {
            float *cp = segu + (size_t)(nseg - 1) * sstride + off;  // pass 1's copy of the initial state
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) *reinterpret_cast<f32x4 *>(cp + 16 * mt) = S[c][mt];
        }
        take_scale(c);
    }

    // ---- prologue: the ring's first NR - 1 chunks, chunk 0's slice blocks
#pragma unroll
    for (int m = 0; m < NR - 1; ++m)
        if (m < NCs) issue(m);
    SR cur[NCH], nxt[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        cur[c].eu = cur[c].eo = 0;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) cur[c].u[tt] = V4{};
        if constexpr (PASS == 1) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) cur[c].o[tt] = V4{};
        }
        nxt[c] = cur[c];
        load_slice(cur[c], c, 0);
    }
    unsigned int nonfinite = 0;

    for (int n = 0; n < NCs; ++n) {
        // chunk n's ring part has landed (this wave's loads: all but the later chunks'; then
        // everyone's, at the barrier), and every wave is done with chunk n - 1's slot
        if (n + NR - 2 < NCs) {
            if (hi)
                wait_vmcnt<Cfg::CNT_HI *(NR - 2)>();
            else
                wait_vmcnt<Cfg::CNT_LO *(NR - 2)>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_lds();
        if (n + 1 < NCs) {
#pragma unroll
            for (int c = 0; c < NCH; ++c) load_slice(nxt[c], c, n + 1);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the slice loads go out before the ring's
        if (n + NR - 1 < NCs) issue(n + NR - 1);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);

        const unsigned char *slot = smem + (n % NR) * SLOT;
        const OH *bWT = reinterpret_cast<const OH *>(slot + Cfg::S_WT);
        const OH *bKH = reinterpret_cast<const OH *>(slot + Cfg::S_KH);
        const float *bG = reinterpret_cast<const float *>(slot + Cfg::S_GAM);
        const int *bScl = reinterpret_cast<const int *>(slot + Cfg::S_SCL);
        const int eW = bScl[0], eK = bScl[2];

        // the state operands (fp16, the chains' scales)
        FH Sh[NCH][NKB];
        int sS0[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            sS0[c] = sS[c];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = S[c][2 * kb + j / 4][j % 4];
                Sh[c][kb] = FH::make(x);
            }
        }
        // P = W S^T, each W^T fragment shared by the wave's chains
        f32x4 P[NCH][NT];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) P[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const FH wf = FH::load_pair(bWT + (kb * NT + tt) * PE, lane);
#pragma unroll
                for (int c = 0; c < NCH; ++c) P[c][tt] = mma(wf, Sh[c][kb], P[c][tt]);
            }
        // U = U~ - W S^T (U~ = 0 for Phi) at the chain's working scale 2^sW, then scaled to fp16 by
        // its wave-wide maximum.  sW is the state's own scale unless U~ is far larger than the state
        // (a state that has decayed to almost nothing), in which case the state is taken down to
        // U~'s scale: every power of two is applied to a value with ldexp, never formed as a factor,
        // so a Phi that decays by e^-75 per token for a whole segment stays exact and finite.
        // In that working scale every factor below is a moderate power of two (at most 2^16 for U~;
        // one that underflows multiplies a term far below the other's rounding).
        FH Uh[NCH][NTKB];
        int sU[NCH], sWk[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int sW = is_phi(c) ? sS[c] : min(sS[c], cur[c].eu + 16);
            sWk[c] = sW;
            const float fU = is_phi(c) ? 0.f : ldexp2(1.f, sW - cur[c].eu), fW = ldexp2(1.f, sW - sS[c] - eW);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) P[c][tt][i] = fmaf((float)cur[c].u[tt][i], fU, -(P[c][tt][i] * fW));
            // U's fp16 scale from bounds, as in the per-slice stage: the stored U~ and W^T blocks
            // are below 2^14 and the chain's state operand below 2^eS, so
            //   |U| < 2^(14 + sW - eu) + 2^(14 + eS + log2 DK + sW - sS - eW)
            // (no U~ term on a transition chain, no W S term while the state is zero)
            constexpr int LOG2DK = DK == 128 ? 7 : 6;
            static_assert(DK == 64 || DK == 128, "dk of 64 or 128");
            const int b1 = is_phi(c) ? ZERO_S : 14 + sW - cur[c].eu;
            const int b2 = eS[c] == ZERO_S ? ZERO_S : 14 + eS[c] + LOG2DK + sW - sS[c] - eW;
            const int bnd = max(b1, b2);
            sU[c] = (F32 || bnd == ZERO_S) ? 0 : 14 - bnd;
#pragma unroll
            for (int kb = 0; kb < NTKB; ++kb) {
                float x[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int t = 2 * kb + j / 4;
                    x[j] = (t < NT) ? ldexp2(P[c][t < NT ? t : 0][j % 4], sU[c]) : 0.f;
                }
                Uh[c][kb] = FH::make(x);
            }
        }
        // S^T <- diag(gamma) S^T + K^^T U, each K^ fragment shared by the wave's chains
        f32x4 A[NCH][NDK];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) A[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NTKB; ++kb)
#pragma unroll
            for (int mt = 0; mt < NDK; ++mt) {
                const FH kf = FH::load_pair(bKH + (kb * NDK + mt) * PE, lane);
#pragma unroll
                for (int c = 0; c < NCH; ++c) A[c][mt] = mma(kf, Uh[c][kb], A[c][mt]);
            }
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if (sWk[c] != sS[c]) {  // the state taken down to the working scale (rare)
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) S[c][mt][i] = ldexp2(S[c][mt][i], sWk[c] - sS[c]);
                sS[c] = sWk[c];
            }
#pragma unroll
        for (int mt = 0; mt < NDK; ++mt) {
            const f32x4 gm = *reinterpret_cast<const f32x4 *>(bG + 16 * mt + 4 * g);
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const float fA = ldexp2(1.f, -(eK + sU[c]));
#pragma unroll
                for (int i = 0; i < 4; ++i) S[c][mt][i] = fmaf(A[c][mt][i], fA, S[c][mt][i] * gm[i]);
            }
        }
        if constexpr (!F32) {  // keep each chain's scaled maximum in [2^11, 2^15)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                float m = 0.f;
#pragma unroll
                for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(S[c][mt][i]));
                if (!wave_max_in(m, 2048.f, 32768.f)) {
                    m = wave_max(m);
                    eS[c] = m == 0.f ? ZERO_S : 15;
                    if (m > 0.f && __builtin_isfinite(m) && (m >= 32768.f || m < 2048.f)) {
                        const int d = pow2_scale(m);
#pragma unroll
                        for (int mt = 0; mt < NDK; ++mt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) S[c][mt][i] = ldexp2(S[c][mt][i], d);
                        sS[c] += d;
                        eS[c] = 14;
                    }
                } else {
                    eS[c] = 15;
                }
            }
        }
        if constexpr (PASS == 1) {
            // O^T = Oi^T + (S^T)^T Qbar^T with the state the chunk started from
            const OH *bQB = reinterpret_cast<const OH *>(slot + Cfg::S_QB);
            const int eQ = bScl[1];
            f32x4 O[NCH][NT];
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) O[c][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const FH qf = FH::load_pair(bQB + (kb * NT + tt) * PE, lane);
#pragma unroll
                    for (int c = 0; c < NCH; ++c) O[c][tt] = mma(Sh[c][kb], qf, O[c][tt]);
                }
            const size_t row0 = (size_t)unit * T + (size_t)(cb + n) * C;
            // the stores, with (COUNT) or without the non-finite count, so that no branch splits them
            auto store = [&](auto count) {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const int j0 = col0(c);
                    const float fO = ldexp2(1.f, -(sS0[c] + eQ)), fI = ldexp2(1.f, -cur[c].eo);
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        f32x4 o;
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] = fmaf(O[c][tt][i], fO, (float)cur[c].o[tt][i] * fI);
                        // lane holds out[token 16 tt + l16][value j0 + 4g + i]
                        E *op = out + (row0 + 16 * tt + l16) * DV + j0 + 4 * g;
                        if constexpr (F32) {
                            *reinterpret_cast<f32x4 *>(op) = o;
                        } else {
                            bf16x4 bo;
#pragma unroll
                            for (int i = 0; i < 4; ++i) bo[i] = (__bf16)o[i];
                            *reinterpret_cast<bf16x4 *>(op) = bo;
#pragma unroll
                            for (int i = 0; i < 4; ++i) o[i] = (float)bo[i];  // what was stored
                        }
                        if constexpr (decltype(count)::value) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) nonfinite += !__builtin_isfinite(o[i]);
                        }
                    }
                }
            };
            if (counts != nullptr)
                store(std::true_type{});
            else
                store(std::false_type{});
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) cur[c] = nxt[c];
    }

    // ---- the chains' end states
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        float *dst = nullptr;
        if (PASS == 0) {
            if (is_phi(c))
                dst = seg > 0 ? phibuf + ((size_t)unit * (nseg - 1) + seg) * pstride : nullptr;
            else
                dst = segu + (size_t)seg * sstride;
        } else if (seg == nseg - 1 && final_state != nullptr) {
            dst = final_state + (size_t)unit * sstride;
        }
        if (dst == nullptr) continue;
        float *fp = dst + lane_off(col0(c));
#pragma unroll
        for (int mt = 0; mt < NDK; ++mt) {
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = ldexp2(S[c][mt][i], -sS[c]);
            *reinterpret_cast<f32x4 *>(fp + 16 * mt) = x;
        }
    }
    if (PASS == 1 && counts != nullptr && nonfinite) atomicAdd(&counts[1], (unsigned long long)nonfinite);
}

// The scan over segments, in fp32: slot j of segbuf goes from segment j's end state from zero to
// segment j + 1's incoming state, X_{j+1} = Phi_j X_j + S_loc_j, for j = 1 .. nseg - 2 (slot 0
// already holds segment 1's incoming state).  One 256-thread work-group per (unit, 16-wide value
// slice); X's slice sits in LDS, Phi_j is read from global memory (every slice of a unit reads
// the same Phi_j), and each wave forms NDK / 4 key tiles with 16x16x4 fp32 MFMAs.
template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_seg_scan_kernel(float *__restrict__ segbuf, const float *__restrict__ phibuf,
                                                          int nseg)
{
    constexpr int NDV = DV / 16, NDK = DK / 16, PX = DK + 4;
    constexpr int MT = NDK / 4;  // key tiles per wave
    __shared__ __attribute__((aligned(16))) float X[16 * PX];  // X~[value][key] of the slice
    const int unit = blockIdx.x / NDV, vs = blockIdx.x % NDV;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
    const int wave = tid >> 6;
    const size_t sstride = (size_t)DV * DK, pstride = (size_t)DK * DK;
    float *segu = segbuf + (size_t)unit * nseg * sstride;
    const float *phu = phibuf + (size_t)unit * (nseg - 1) * pstride;
    for (int e = tid; e < 16 * DK; e += 256) X[(e / DK) * PX + e % DK] = segu[(size_t)(16 * vs + e / DK) * DK + e % DK];
    __syncthreads();
    // this lane's operands of step j: Phi_j[16 mt + l16][4 s + g] for its key tiles, and S_loc_j
    constexpr int NS4 = DK / 4;
    float a_cur[MT][NS4], a_nxt[MT][NS4];
    f32x4 l_cur[MT], l_nxt[MT];
    auto fetch = [&](int j, float (&a)[MT][NS4], f32x4 (&l)[MT]) {
        const float *ph = phu + (size_t)j * pstride;  // ph[c][r] = Phi[r][c]
        const float *sj = segu + (size_t)j * sstride;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int mt = wave + 4 * t;
#pragma unroll
            for (int s = 0; s < NS4; ++s) a[t][s] = ph[(size_t)(4 * s + g) * DK + 16 * mt + l16];
            l[t] = *reinterpret_cast<const f32x4 *>(sj + (size_t)(16 * vs + l16) * DK + 16 * mt + 4 * g);
        }
    };
    if (nseg > 2) fetch(1, a_cur, l_cur);
    for (int j = 1; j + 1 < nseg; ++j) {
        if (j + 2 < nseg) fetch(j + 1, a_nxt, l_nxt);  // in flight while step j computes
        float *sj = segu + (size_t)j * sstride;
        f32x4 acc[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int mt = wave + 4 * t;
            // lane holds Y[key 16 mt + 4g + i][value 16 vs + l16], stored at sj[value][key]
            acc[t] = l_cur[t];
#pragma unroll
            for (int s = 0; s < NS4; ++s) acc[t] = mma4(a_cur[t][s], X[l16 * PX + 4 * s + g], acc[t]);
            *reinterpret_cast<f32x4 *>(sj + (size_t)(16 * vs + l16) * DK + 16 * mt + 4 * g) = acc[t];
        }
        __syncthreads();  // every wave has read X
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int mt = wave + 4 * t;
            *reinterpret_cast<f32x4 *>(X + l16 * PX + 16 * mt + 4 * g) = acc[t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            l_cur[t] = l_nxt[t];
#pragma unroll
            for (int s = 0; s < NS4; ++s) a_cur[t][s] = a_nxt[t][s];
        }
    }
}

}  // namespace kda
