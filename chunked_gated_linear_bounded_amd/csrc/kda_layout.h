// Per-chunk workspace layout shared by the chunk-parallel stage (producer) and
// the sequential state stage (consumer).  Host and device both include it.
//
// Every operand is stored as 16x16 tiles in "accumulator fragment order": tile
// element (row 4*(l/16)+i, column l%16) sits at lane l, slot i (i = 0..3), so
// lane l's four values are contiguous and a wave stores or loads a whole tile
// with one coalesced access per lane.
//
// Per (batch, head, chunk) record, in this order:
//   WT  : W^T    (dk x C)  tiles [ct][rt]  bf16           W = T diag(beta) (K e^G)
//   QBT : Qbar^T (dk x C)  tiles [ct][rt]  fp16, scaled   Qbar = Q e^G - M W
//   KH  : K^     (C x dk)  tiles [st][ct]  fp16, scaled   K^ = K e^(G_last - G)
//   GAM : e^(G_last)       dk float32
//   SCL : 4 int32: the power-of-two exponents QBT and KH are scaled by, 0, 0
// (with fp32 I/O every operand is fp32 and the exponents are 0)
//   then, for each 16-wide slice vt of the value dimension (contiguous):
//   UT  : U~     (C x 16)  tiles [rt]      float32        U~ = T diag(beta) V
//   OIT : Oi^T   (16 x C)  tiles [rt]      float32        Oi = M U~ (intra-chunk output)
// The first four are "region 1" (read by every slice's consumer); a consumer
// that owns slice vt reads region 1 plus its own slice: two byte ranges.
#pragma once
#include <stddef.h>

struct KdaLayout {
    int NT, NDK, NDV;          // C/16, dk/16, dv/16
    size_t tile;               // bytes per 16x16 operand-type tile
    size_t tile32;             // bytes per 16x16 float32 tile (1024)
    size_t wt, qbt, kh, gam, scl;  // byte offsets inside one record
    size_t region1;            // bytes of WT..GAM
    size_t slice;              // bytes of one value slice (UT + OIT)
    size_t ut, oit;            // offsets of UT and OIT inside a slice
    size_t stride;             // bytes per record (256-byte multiple)
};

static inline constexpr KdaLayout kda_layout(int C, int DK, int DV, int esize)
{
    KdaLayout L{};
    L.NT = C / 16;
    L.NDK = DK / 16;
    L.NDV = DV / 16;
    L.tile = (size_t)256 * (size_t)esize;
    L.tile32 = 1024;
    L.wt = 0;
    L.qbt = L.wt + (size_t)L.NDK * L.NT * L.tile;
    L.kh = L.qbt + (size_t)L.NDK * L.NT * L.tile;
    L.gam = L.kh + (size_t)L.NT * L.NDK * L.tile;
    L.scl = L.gam + (size_t)DK * 4;
    L.region1 = L.scl + 16;
    L.ut = 0;
    L.oit = (size_t)L.NT * L.tile32;
    L.slice = 2 * (size_t)L.NT * L.tile32;
    size_t end = L.region1 + (size_t)L.NDV * L.slice;
    L.stride = (end + 255) / 256 * 256;
    return L;
}
