// Per-chunk workspace layout shared by the chunk-parallel stage (producer) and
// the sequential state stage (consumer).  Host and device both include it.
//
// Operands are 16x16 tiles of an accumulator ("D") layout: tile element
// (row 4*(l/16)+i, column l%16) belongs to lane l, slot i (i = 0..3).
//
// Operand blocks the consumer feeds to MFMAs (WT, QBT, KH) are stored as tile
// PAIRS: the two tiles (2p, c) and (2p+1, c) that make one 32-deep K-block are
// interleaved per lane, lane l's 8 values contiguous (slots 0-3 from tile 2p,
// 4-7 from tile 2p+1).  A wave loads one MFMA operand fragment with a single
// 16-byte read per lane.  UT and OIT are plain tiles (lane l's 4 values contiguous).
//
// Per (batch, head, chunk) record, in this order:
//   WT  : W^T    (dk x C)  pairs [ct/2][rt]     16-bit, scaled   W = T diag(beta) (K e^G)
//   QBT : Qbar^T (dk x C)  pairs [ct/2][rt]     16-bit, scaled   Qbar = Q e^G - M W
//   KH  : K^     (C x dk)  pairs [st/2][ct]     16-bit, scaled   K^ = K e^(G_last - G)
//   GAM : e^(G_last)       dk float32
//   SCL : 4 int32: the power-of-two exponents WT, QBT and KH are scaled by, 0
//   then, for each 16-wide slice vt of the value dimension (contiguous):
//   SSC : 4 int32: the power-of-two exponents UT and OIT are scaled by, 0, 0
//   UT  : U~     (C x 16)  tiles [rt]   16-bit, scaled   U~ = T diag(beta) V
//   OIT : Oi^T   (16 x C)  tiles [rt]   16-bit, scaled   Oi = M U~ (intra-chunk output)
// 16-bit means fp16 for bf16 I/O; with fp32 I/O these blocks are fp32 and the
// exponents are 0.  The first five blocks are "region 1" (read by every
// slice's consumer); a consumer that owns slice vt reads region 1 plus its own
// slice: two contiguous byte ranges.
#pragma once
#include <stddef.h>

struct KdaLayout {
    int NT, NDK, NDV;              // C/16, dk/16, dv/16
    int NTP;                       // token tile pairs, ceil(NT/2)
    size_t tile;                   // bytes per 16x16 operand-type tile
    size_t wt, qbt, kh, gam, scl;  // byte offsets inside one record
    size_t region1;                // bytes of WT..SCL
    size_t slice;                  // bytes of one value slice (SSC + UT + OIT)
    size_t ssc, ut, oit;           // offsets of SSC, UT and OIT inside a slice
    size_t stride;                 // bytes per record (256-byte multiple)
};

static inline constexpr KdaLayout kda_layout(int C, int DK, int DV, int esize)
{
    KdaLayout L{};
    L.NT = C / 16;
    L.NDK = DK / 16;
    L.NDV = DV / 16;
    L.NTP = (L.NT + 1) / 2;
    L.tile = (size_t)256 * (size_t)esize;
    L.wt = 0;
    L.qbt = L.wt + (size_t)L.NDK * L.NT * L.tile;
    L.kh = L.qbt + (size_t)L.NDK * L.NT * L.tile;
    L.gam = L.kh + (size_t)2 * L.NTP * L.NDK * L.tile;
    L.scl = L.gam + (size_t)DK * 4;
    L.region1 = L.scl + 16;
    L.ssc = 0;
    L.ut = 16;
    L.oit = L.ut + (size_t)L.NT * L.tile;
    L.slice = L.oit + (size_t)L.NT * L.tile;
    size_t end = L.region1 + (size_t)L.NDV * L.slice;
    L.stride = (end + 255) / 256 * 256;
    return L;
}

// ---------------------------------------------------------------- segmented state stage
// The sequential stage can cut each head's sequence into segments walked side by side, so that a
// head with thousands of chunks is not carried by one serial chain.  Writing one chunk's state
// update as the affine map  S^T <- A_c S^T + B_c  (A_c = diag(gamma) - K^^T W, dk x dk), a segment
// maps its incoming state X to  Phi X + S_loc,  where Phi is the product of its A_c and S_loc is
// the state it ends in from zero.  Pass 0 forms both per segment (the first segment's end state
// directly, from the true initial state); a scan over the segments gives each segment's incoming
// state; pass 1 walks every segment again from that state and writes the outputs.
//
// What one LDS ring slot holds per chunk: pass 0 reads W^T, then K^, gamma and the exponents
// (two byte ranges of the record); pass 1 reads region 1 as stored.
struct KdaSegRing {
    int p1_src, p1_len;  // first range: offset in the record, bytes
    int p2_src, p2_len;  // second range (pass 0 only), placed right after the first in the slot
    int slot;            // bytes per slot (16-byte multiple)
    int depth;           // slots in the ring (0: does not fit twice)
    int ndma;            // 1 KiB direct-load instructions per chunk
};

static inline constexpr KdaSegRing kda_seg_ring(const KdaLayout &L, int pass)
{
    KdaSegRing r{};
    if (pass) {
        r.p1_src = 0;
        r.p1_len = (int)L.region1;
    } else {
        r.p1_src = (int)L.wt;
        r.p1_len = (int)(L.qbt - L.wt);
        r.p2_src = (int)L.kh;
        r.p2_len = (int)(L.region1 - L.kh);
    }
    r.slot = (r.p1_len + r.p2_len + 15) / 16 * 16;
    const int lds = 160 * 1024;
    r.depth = 4 * r.slot <= lds ? 4 : 3 * r.slot <= lds ? 3 : 2 * r.slot <= lds ? 2 : 0;
    r.ndma = (r.p1_len + 1023) / 1024 + (r.p2_len + 1023) / 1024;
    return r;
}

// Work-groups of the segmented passes have four waves; each issues every fourth direct load of a
// chunk and waits for its own with a partial vmcnt, which must fit the 6-bit counter.
static inline constexpr bool kda_seg_ring_ok(const KdaSegRing &r)
{
    return r.depth >= 2 && ((r.ndma + 3) / 4) * (r.depth - 2) <= 63;
}

static inline constexpr bool kda_seg_supported(const KdaLayout &L)
{
    return kda_seg_ring_ok(kda_seg_ring(L, 0)) && kda_seg_ring_ok(kda_seg_ring(L, 1));
}

// Segments per head: enough (head, segment) work-groups to give each of the 256 compute units one,
// at least 8 chunks per segment, and no empty segment.
static inline constexpr int kda_seg_count(long long units, int nc)
{
    if (units <= 0 || units >= 256 || nc < 16) return 1;
    long long s = 256 / units;
    if (s > nc / 8) s = nc / 8;
    if (s < 1) s = 1;
    const long long len = (nc + s - 1) / s;
    return (int)((nc + len - 1) / len);
}

// Which state stage a fixed-length forward runs.  The per-slice stage (kda_state.h) gives each
// (head, 16-wide value slice) one work-group walking the whole sequence: where those work-groups
// fill the 256 compute units it is the faster of the two (it moves each record once and its chain
// is short).  Where they do not -- fewer than 256 / (dv / 16) heads -- the segmented stage cuts the
// sequence so that 256 work-groups run; with 256 heads or more it runs one segment (pass 1 alone,
// one work-group per head instead of dv / 16 rounds of per-slice work-groups).
static inline constexpr bool kda_use_segmented(const KdaLayout &L, long long units)
{
    return kda_seg_supported(L) && (units * L.NDV < 256 || units >= 256);
}

// The whole forward workspace: the records [unit][chunk], then (segments > 1) the segment states
// [unit][nseg][dv][dk] fp32 (slot j < nseg - 1: segment j's end state from pass 0, after the scan
// segment j + 1's incoming state; slot nseg - 1: a copy of the initial state) and the segment
// transitions [unit][nseg - 1][dk][dk] fp32 (slot j = Phi of segment j, stored transposed; slot 0
// unused).
struct KdaFwdPlan {
    bool segmented;  // the state stage runs kda_state_seg.h (else the per-slice stage)
    int nseg, seglen;
    size_t rec_bytes, seg_off, phi_off, total;
};

static inline constexpr KdaFwdPlan kda_fwd_plan(int B, int H, int T, int C, int dk, int dv, int esize)
{
    KdaFwdPlan p{};
    const KdaLayout L = kda_layout(C, dk, dv, esize);
    const long long units = (long long)B * H;
    const int nc = T / C;
    p.rec_bytes = (size_t)units * (size_t)nc * L.stride;
    p.segmented = kda_use_segmented(L, units);
    p.nseg = p.segmented ? kda_seg_count(units, nc) : 1;
    p.seglen = p.nseg > 0 && nc > 0 ? (nc + p.nseg - 1) / p.nseg : nc;
    p.seg_off = p.rec_bytes;
    p.phi_off = p.seg_off;
    p.total = p.rec_bytes;
    if (p.nseg > 1) {
        p.phi_off = p.seg_off + (size_t)units * p.nseg * (size_t)dv * dk * 4;
        p.total = p.phi_off + (size_t)units * (p.nseg - 1) * (size_t)dk * dk * 4;
    }
    return p;
}
