// Internal interface between the host C ABI (kda_abi.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime_api.h>

namespace kda {

struct LaunchArgs {
    const void *q, *k, *v, *a, *beta;
    float g_min;
    int logsig;                 // 0: bounded gate, 1: log-sigmoid (ablation)
    int chunk, B, H, T, dk, dv;
    bool fp32;                  // I/O element type fp32 (else bf16)
    void *out;
    float *final_state;
    const float *init_state;    // nullable: S_0 of the chunked forward
    float *state;               // decode: the state, updated in place
    void *workspace;
    float *G_out;
    unsigned long long *counts;
    hipStream_t stream;
    // a window of the sequence (fixed-length batches): chunks c0 .. c0 + ncw - 1 of every head, whose
    // records sit in the workspace as [B*H][ncw]; ncw = 0 means the whole sequence (c0 = 0)
    int c0, ncw;
    // packed documents (NULL cu: fixed-length batch)
    const int *cu;              // device cu_seqlens[nseq + 1]
    int nseq;                   // documents
    int ncmax;                  // chunk records per head: T / chunk + nseq
    int nrun;                   // runs of documents the state stage walks (one work-group each per head and slice)
    size_t plan_offset;         // byte offset of the plan tables in the workspace
    // gate pre-activation from a rank-`rank` factor (NULL lr_h: read from a)
    const void *lr_h, *lr_z;    // [B][T][rank], [H][dk][rank] (I/O element type)
    const float *lr_A;          // [H][dk]
    int rank;                   // 16, 32, 64 or 128
    // backward
    float *states;              // nullable: chunk start states [B*H][NC][dv][dk] (state stage)
    float *dstates;             // gradients of the chunk end states, same layout
    const void *dout;           // [B][H][T][dv] (I/O element type)
    const float *dfinal;        // nullable: gradient of final_state
    float *dq, *dk_, *dv_, *da, *dbeta, *dinit;  // float32 gradients (dinit nullable)
};

hipError_t launch_intra(const LaunchArgs &p);  // chunk-parallel stage -> workspace
hipError_t launch_intra_lowrank(const LaunchArgs &p);  // the same, gate pre-activation from lr_h, lr_z, lr_A
hipError_t launch_state(const LaunchArgs &p);  // sequential stage: workspace -> out, final state
hipError_t launch_gate_cumsum(const LaunchArgs &p);
hipError_t launch_decode(const LaunchArgs &p);  // one token per head, state in place
hipError_t launch_bwd(const LaunchArgs &p);     // gradients (recompute, reverse state pass, chunk stage)
hipError_t noalloc_scratch(void **ptr);         // this device's scratch of kda_chunk_fwd_noalloc
hipError_t launch_state_fill(float *dst, const float *src, size_t n, hipStream_t stream);  // dst = src or 0

}  // namespace kda
