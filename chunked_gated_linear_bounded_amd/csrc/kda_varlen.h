// Packed sequences: several documents of different lengths laid end to end in one
// token stream, each run through the recurrence from its own initial state with
// nothing carried across a document boundary (packing many short documents into
// one long training sequence: "Breaking Through Trillion-Parameter Multimodal MoE:
// Key Innovations from Ultra-Long Context to Extreme Sparsity", sec. 3, the
// 256K-1M context phase).
//
// Document i covers tokens [cu[i], cu[i+1]) of the stream.  It is cut into
// ceil(len_i / C) chunks; the last one may be short.  A short chunk is padded to
// C rows with q = k = 0, beta = 0 and g = 0, which leaves every product of the
// chunk form exactly what the shorter chunk gives (zero rows and columns of A and
// M, identity rows of T, a flat prefix sum G so e^(G_last) is the decay up to the
// last real row), and the padded rows' outputs are not stored.
//
// The two plan kernels below turn cu into the tables both stages index by; they run ahead
// of them on the same stream (the first writes bnd and coff, the second the rest):
//   bnd[i]  (i = 0..N)    document boundaries, made nondecreasing and clipped to [0, T]
//   coff[i] (i = 0..N)    index of document i's first chunk; coff[N] = chunks in use
//   ctab[j] (j < NCmax)   {first token, rows, document, flags} of chunk j (flags: bit 0 = the
//                         document's first chunk, bit 1 = its last; on a last chunk, bits 2.. =
//                         1 + the document of the next chunk, 0 if there is none); rows = 0
//                         past the last chunk
//   seg[p]  (p = 0..P)    the documents split into P runs of about equal chunk counts: run p
//                         is documents seg[p] .. seg[p+1]-1, chunks coff[seg[p]] .. coff[seg[p+1]]-1
// With the boundaries nondecreasing inside [0, T] the chunk count is at most
// floor(T / C) + N = NCmax, the number of records the workspace holds, so no
// content of cu can make a stage index outside its buffers.
#pragma once
#include "kda_device.h"

namespace kda {

// Inclusive scan over the work-group (sum, or maximum of nonnegative values); `total`
// receives the reduction over all threads.
template <bool MAX>
__device__ __forceinline__ int block_scan(int x, int *red, int &total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x = MAX ? (x > y ? x : y) : x + y;
    }
    if (lane == 63) red[w] = x;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int u = 0; u < nw; ++u) {
        const int r = red[u];
        if (u < w) before = MAX ? (before > r ? before : r) : before + r;
        total = MAX ? (total > r ? total : r) : total + r;
    }
    __syncthreads();  // red is reused by the next scan
    return MAX ? (before > x ? before : x) : before + x;
}

template <int C>
__global__ __launch_bounds__(1024) void kda_varlen_plan_kernel(const int *__restrict__ cu, int N, int T, int NCmax,
                                                              int *__restrict__ bnd, int *__restrict__ coff)
{
    __shared__ int red[16];
    const int tid = threadIdx.x;
    auto clip = [T](int x) { return x < 0 ? 0 : (x > T ? T : x); };
    int cmax = 0, csum = 0;  // running maximum of the clipped boundaries; chunks of earlier tiles
    for (int base = 0; base < N; base += 1024) {
        const int i = base + tid;
        const bool doc = i < N;
        const int e0 = doc ? clip(cu[i]) : 0, e1 = doc ? clip(cu[i + 1]) : 0;
        int tmax, tsum;
        const int s0 = max(cmax, block_scan<true>(e0, red, tmax));  // start of document i
        const int s1 = max(s0, e1);                                  // its end
        const int len = doc ? s1 - s0 : 0;
        const int nch = (len + C - 1) / C;
        const int c0 = csum + block_scan<false>(nch, red, tsum) - nch;
        if (doc) {
            bnd[i] = s0;
            coff[i] = c0;
        }
        cmax = max(cmax, tmax);
        csum += tsum;
    }
    if (tid == 0) {
        bnd[N] = max(cmax, clip(cu[N]));
        coff[N] = min(csum, NCmax);
    }
}

// The document that chunk j (< coff[N]) belongs to: the last i with coff[i] <= j.  Documents
// without chunks share their offset with the next one, so the search lands on a document
// that has tokens.
__device__ __forceinline__ int doc_of_chunk(const int *__restrict__ coff, int N, int j) {
    int lo = 0, hi = N + 1;  // first index with coff[index] > j lies in (0, N]
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (coff[mid] > j) hi = mid;
        else lo = mid + 1;
    }
    return lo - 1;
}

// Second plan kernel (after the first): block 0 splits the documents into P runs of about equal
// chunk counts (seg); blocks 1 .. NB write the chunk table, one entry per thread, so a long
// document costs no more than many short ones; block 1 + NB + i gives document i, if it has no
// tokens, its final state (its initial state, else zero) for every head, since no chunk of the
// state stage will.
template <int C>
__global__ __launch_bounds__(256) void kda_varlen_seg_kernel(const int *__restrict__ bnd, const int *__restrict__ coff,
                                                             int N, int P, int NCmax, int *__restrict__ seg,
                                                             int4 *__restrict__ ctab, int NB, const float *init,
                                                             float *final_state, int per_doc) {
    const int tid = threadIdx.x;
    if (blockIdx.x >= 1 && blockIdx.x <= NB) {
        const int j = (blockIdx.x - 1) * 256 + tid, ntot = coff[N];
        if (j >= NCmax) return;
        int4 e = make_int4(0, 0, 0, 0);
        if (j < ntot) {
            const int i = doc_of_chunk(coff, N, j), m = j - coff[i], nch = coff[i + 1] - coff[i];
            const int len = bnd[i + 1] - bnd[i];
            int flags = (m == 0 ? 1 : 0) | (m == nch - 1 ? 2 : 0);
            if (m == nch - 1 && j + 1 < ntot) flags |= (doc_of_chunk(coff, N, j + 1) + 1) << 2;
            e = make_int4(bnd[i] + m * C, min(C, len - m * C), i, flags);
        }
        ctab[j] = e;
        return;
    }
    if (blockIdx.x == 0) {
        const long long ntot = coff[N];
        for (int p = tid; p <= P; p += 256) {
            const long long target = (ntot * p + P - 1) / P;
            int lo = 0, hi = N;  // lowest i with coff[i] >= target (coff is nondecreasing, coff[N] = ntot)
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (coff[mid] >= target) hi = mid;
                else lo = mid + 1;
            }
            seg[p] = p == 0 ? 0 : (p == P ? N : lo);
        }
        return;
    }
    const int i = blockIdx.x - 1 - NB;
    if (final_state == nullptr || bnd[i + 1] != bnd[i]) return;
    float *dst = final_state + (size_t)i * per_doc;
    const float *src = init == nullptr ? nullptr : init + (size_t)i * per_doc;
    for (int e = tid; e < per_doc; e += 256) dst[e] = src == nullptr ? 0.f : src[e];
}

}  // namespace kda
