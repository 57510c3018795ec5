// Per-chunk workspace layout shared by the chunk-parallel stage (producer) and
// the sequential state stage (consumer).  Host and device both include it.
//
// Every operand is stored as 16x16 tiles in "accumulator fragment order": tile
// element (row 4*(l/16)+i, column l%16) sits at lane l, slot i (i = 0..3), so
// lane l's four values are contiguous and a wave stores or loads a whole tile
// with one coalesced 8-byte (bf16) or 16-byte (fp32) access per lane.
//
// Per (batch, head, chunk) record, in this order:
//   WT  : W^T   (dk x C)  tiles [ct][rt]       W = T diag(beta) (K * e^G)
//   QT  : Q~^T  (dk x C)  tiles [ct][rt]       Q~ = Q * e^G
//   KH  : K^    (C x dk)  tiles [st][ct]       K^ = K * e^(G_last - G)
//   MT  : M^T   (C x C)   causal tiles only, index rt*(rt+1)/2 + st (st <= rt)
//   GAM : e^(G_last)  dk float32
//   UT  : U~    (C x dv)  tiles [vt][rt]       U~ = T diag(beta) V
// The first five are contiguous ("region 1"), then the dv/16 column slices of
// U~ each contiguous, so a consumer that owns one 16-wide slice of the value
// dimension reads two contiguous byte ranges per chunk.
#pragma once
#include <stddef.h>

struct KdaLayout {
    int NT, NDK, NDV, NMT;     // C/16, dk/16, dv/16, causal tile count
    size_t tile;               // bytes per 16x16 tile
    size_t wt, qt, kh, mt, gam, ut;  // byte offsets inside one record
    size_t region1;            // bytes of WT..GAM
    size_t uslice;             // bytes of one 16-wide U~ slice (NT tiles)
    size_t stride;             // bytes per record (256-byte multiple)
};

static inline constexpr KdaLayout kda_layout(int C, int DK, int DV, int esize)
{
    KdaLayout L{};
    L.NT = C / 16;
    L.NDK = DK / 16;
    L.NDV = DV / 16;
    L.NMT = L.NT * (L.NT + 1) / 2;
    L.tile = (size_t)256 * (size_t)esize;
    L.wt = 0;
    L.qt = L.wt + (size_t)L.NDK * L.NT * L.tile;
    L.kh = L.qt + (size_t)L.NDK * L.NT * L.tile;
    L.mt = L.kh + (size_t)L.NT * L.NDK * L.tile;
    L.gam = L.mt + (size_t)L.NMT * L.tile;
    L.region1 = L.gam + (size_t)DK * 4;
    L.ut = L.region1;
    L.uslice = (size_t)L.NT * L.tile;
    size_t end = L.ut + (size_t)L.NDV * L.uslice;
    L.stride = (end + 255) / 256 * 256;
    return L;
}
