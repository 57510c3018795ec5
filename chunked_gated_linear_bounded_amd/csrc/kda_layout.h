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
