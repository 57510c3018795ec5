// Host side of the C ABI declared in include/kda.h: argument validation (pure
// host code, no HIP call before every check has passed), workspace sizing and
// dispatch to the kernel launchers.
#include <math.h>
#include <stdint.h>

#include "kda.h"
#include "kda_launch.h"
#include "kda_layout.h"

namespace {

bool aligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int check_shape(int B, int H, int T, int dk, int dv, int chunk, int io) {
    if (io != KDA_BF16 && io != KDA_FP32) return KDA_ERR_DTYPE;
    if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_CHUNK;
    if (B < 1 || H < 1 || T < 0) return KDA_ERR_SHAPE;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_SHAPE;
    if (T % chunk != 0) return KDA_ERR_SHAPE;
    if (H > 65535 || B > 65535) return KDA_ERR_SHAPE;  // grid y and z of the chunk stage
    const double elems = (double)B * H * (double)T * (dk > dv ? dk : dv);
    if (elems >= 1099511627776.0) return KDA_ERR_SHAPE;  // 2^40
    return KDA_OK;
}

int check_gate(float g_min, int gate_mode) {
    if (gate_mode != KDA_GATE_BOUNDED && gate_mode != KDA_GATE_LOGSIGMOID) return KDA_ERR_MODE;
    if (gate_mode == KDA_GATE_BOUNDED) {
        if (!isfinite(g_min) || !(g_min < 0.0f) || g_min < KDA_G_MIN_LOWEST) return KDA_ERR_GMIN;
    }
    return KDA_OK;
}

// the chunk records and, when the state stage runs in segments, the segments' states and maps
size_t workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int io) {
    return kda_fwd_plan(B, H, T, chunk, dk, dv, io == KDA_FP32 ? 4 : 2).total;
}

int check_ptrs_ws(int B, int H, int T, int dk, int dv, int chunk, int io, const void *workspace,
                  size_t workspace_bytes_given) {
    const size_t need = workspace_bytes(B, H, T, dk, dv, chunk, io);
    if (need > 0) {
        if (!workspace || workspace_bytes_given < need) return KDA_ERR_WORKSPACE;
        if (!aligned(workspace, 16)) return KDA_ERR_ALIGN;
    }
    return KDA_OK;
}

// The gate pre-activation from a rank-R factor instead of the a tensor (NULL h: read a).
struct LowRank {
    bool on;
    const void *h, *z;
    const float *A;
    int rank;
};

int intra_impl(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
               int chunk, int B, int H, int T, int dk, int dv, int io, void *workspace,
               size_t workspace_bytes_given, hipStream_t stream, int gate_mode, unsigned long long *counts,
               bool launch, const LowRank &lr = LowRank{false, nullptr, nullptr, nullptr, 0}) {
    int st = check_shape(B, H, T, dk, dv, chunk, io);
    if (st != KDA_OK) return st;
    st = check_gate(g_min, gate_mode);
    if (st != KDA_OK) return st;
    const bool low = lr.on;
    if (low && lr.rank != 16 && lr.rank != 32 && lr.rank != 64 && lr.rank != 128) return KDA_ERR_SHAPE;
    if (T > 0 && (!q || !k || !v || !beta)) return KDA_ERR_NULL;  // empty arrays may be NULL
    if (T > 0 && (low ? (!lr.h || !lr.z || !lr.A) : !a)) return KDA_ERR_NULL;
    const size_t esz = io == KDA_FP32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(a, 16) || !aligned(beta, esz) ||
        !aligned(lr.h, 16) || !aligned(lr.z, 16) || !aligned(lr.A, 4) || (counts && !aligned(counts, 8)))
        return KDA_ERR_ALIGN;
    st = check_ptrs_ws(B, H, T, dk, dv, chunk, io, workspace, workspace_bytes_given);
    if (st != KDA_OK || !launch || T == 0) return st;
    kda::LaunchArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
    p.g_min = g_min;
    p.logsig = gate_mode == KDA_GATE_LOGSIGMOID;
    p.chunk = chunk; p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = dv;
    p.fp32 = io == KDA_FP32;
    p.workspace = workspace; p.counts = counts; p.stream = stream;
    if (low) {
        p.a = nullptr;
        p.lr_h = lr.h; p.lr_z = lr.z; p.lr_A = lr.A; p.rank = lr.rank;
    }
    return kda::launch_intra(p) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int state_impl(const void *workspace, size_t workspace_bytes_given, int chunk, int B, int H, int T, int dk,
               int dv, int io, void *out, float *final_state, hipStream_t stream, unsigned long long *counts,
               const float *init_state, bool launch) {
    int st = check_shape(B, H, T, dk, dv, chunk, io);
    if (st != KDA_OK) return st;
    if (T > 0 && !out) return KDA_ERR_NULL;  // an empty out may be NULL
    if (!aligned(out, 16) || (final_state && !aligned(final_state, 16)) || (counts && !aligned(counts, 8)) ||
        (init_state && !aligned(init_state, 16)))
        return KDA_ERR_ALIGN;
    st = check_ptrs_ws(B, H, T, dk, dv, chunk, io, workspace, workspace_bytes_given);
    if (st != KDA_OK || !launch) return st;
    if (T == 0) {  // empty sequence: no output rows, the state is the initial one
        const size_t bytes = (size_t)B * H * dv * dk * sizeof(float);
        if (final_state && !init_state && hipMemsetAsync(final_state, 0, bytes, stream) != hipSuccess)
            return KDA_ERR_HIP;
        if (final_state && init_state && final_state != init_state &&
            hipMemcpyAsync(final_state, init_state, bytes, hipMemcpyDeviceToDevice, stream) != hipSuccess)
            return KDA_ERR_HIP;
        return KDA_OK;
    }
    kda::LaunchArgs p{};
    p.chunk = chunk; p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = dv;
    p.fp32 = io == KDA_FP32;
    p.out = out; p.final_state = final_state; p.init_state = init_state;
    p.workspace = const_cast<void *>(workspace);
    p.counts = counts; p.stream = stream;
    return kda::launch_state(p) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int fwd_impl(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
             int chunk, int B, int H, int T, int dk, int dv, int io, void *out, float *final_state,
             void *workspace, size_t workspace_bytes_given, hipStream_t stream, int gate_mode,
             unsigned long long *counts, const float *init_state,
             const LowRank &lr = LowRank{false, nullptr, nullptr, nullptr, 0}) {
    // validate both stages before launching either
    int st = intra_impl(q, k, v, a, beta, g_min, chunk, B, H, T, dk, dv, io, workspace, workspace_bytes_given,
                        stream, gate_mode, counts, false, lr);
    if (st != KDA_OK) return st;
    st = state_impl(workspace, workspace_bytes_given, chunk, B, H, T, dk, dv, io, out, final_state, stream,
                    counts, init_state, false);
    if (st != KDA_OK) return st;
    st = intra_impl(q, k, v, a, beta, g_min, chunk, B, H, T, dk, dv, io, workspace, workspace_bytes_given,
                    stream, gate_mode, counts, true, lr);
    if (st != KDA_OK) return st;
    return state_impl(workspace, workspace_bytes_given, chunk, B, H, T, dk, dv, io, out, final_state, stream,
                      counts, init_state, true);
}

// The allocation-free forward: windows of chunks whose records fit the static scratch, each a
// chunk stage and a state stage launch; the state goes from window to window through final_state
// (else the scratch's first bytes).  All checks run before the first HIP call.
int noalloc_impl(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
                 int chunk, int B, int H, int T, int dk, int dv, int io, void *out, float *final_state,
                 hipStream_t stream, int gate_mode, unsigned long long *counts, const float *init_state) {
    int st = check_shape(B, H, T, dk, dv, chunk, io);
    if (st != KDA_OK) return st;
    st = check_gate(g_min, gate_mode);
    if (st != KDA_OK) return st;
    if (T > 0 && (!q || !k || !v || !a || !beta || !out)) return KDA_ERR_NULL;  // empty arrays may be NULL
    const size_t esz = io == KDA_FP32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(a, 16) || !aligned(beta, esz) ||
        !aligned(out, 16) || (final_state && !aligned(final_state, 16)) || (init_state && !aligned(init_state, 16)) ||
        (counts && !aligned(counts, 8)))
        return KDA_ERR_ALIGN;
    const KdaLayout L = kda_layout(chunk, dk, dv, (int)esz);
    const size_t nstate = (size_t)B * H * dv * dk;
    const size_t state_bytes = final_state ? 0 : (nstate * sizeof(float) + 255) / 256 * 256;
    const size_t per_chunk = (size_t)B * H * L.stride;  // one chunk of every head
    if (state_bytes + per_chunk > (size_t)KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    void *scr = nullptr;
    if (kda::noalloc_scratch(&scr) != hipSuccess) return KDA_ERR_HIP;
    float *carrier = final_state ? final_state : reinterpret_cast<float *>(scr);
    if (T == 0)  // the state of an empty sequence is the initial one
        return kda::launch_state_fill(carrier, init_state, final_state ? nstate : 0, stream) == hipSuccess
                   ? KDA_OK : KDA_ERR_HIP;
    const int NC = T / chunk;
    const size_t fit = ((size_t)KDA_NOALLOC_SCRATCH_BYTES - state_bytes) / per_chunk;
    const int ncw = fit < (size_t)NC ? (int)fit : NC;
    kda::LaunchArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
    p.g_min = g_min;
    p.logsig = gate_mode == KDA_GATE_LOGSIGMOID;
    p.chunk = chunk; p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = dv;
    p.fp32 = io == KDA_FP32;
    p.out = out; p.final_state = carrier;
    p.workspace = static_cast<unsigned char *>(scr) + state_bytes;
    p.counts = counts; p.stream = stream;
    for (int c0 = 0; c0 < NC; c0 += ncw) {
        p.c0 = c0;
        p.ncw = NC - c0 < ncw ? NC - c0 : ncw;
        p.init_state = c0 == 0 ? init_state : carrier;
        if (kda::launch_intra(p) != hipSuccess) return KDA_ERR_HIP;
        if (kda::launch_state(p) != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

// Packed documents: chunk records per head (an upper bound on the chunks the documents
// can need, whatever cu_seqlens holds), and where the plan tables start.
struct VarlenSizes {
    long long ncmax;
    int nrun;  // runs of documents: enough (document, head, slice) walks to give every CU one, at most N
    size_t plan_offset, total;
};

int check_varlen(int N, int H, int T, int dk, int dv, int chunk, int io, VarlenSizes *vs) {
    if (io != KDA_BF16 && io != KDA_FP32) return KDA_ERR_DTYPE;
    if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_CHUNK;
    if (N < 1 || H < 1 || T < 0) return KDA_ERR_SHAPE;
    if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return KDA_ERR_SHAPE;
    if (H > 65535) return KDA_ERR_SHAPE;
    const long long ncmax = (long long)(T / chunk) + N;
    if (ncmax > 2147483647LL - 1024) return KDA_ERR_SHAPE;
    if ((long long)N * H * (dv / 16) + 8LL * (dv / 16) > 2147483647LL) return KDA_ERR_SHAPE;  // state grid
    const double elems = (double)H * (double)T * (dk > dv ? dk : dv);
    if (elems >= 1099511627776.0) return KDA_ERR_SHAPE;  // 2^40
    const KdaLayout L = kda_layout(chunk, dk, dv, io == KDA_FP32 ? 4 : 2);
    const long long units = (long long)H * (dv / 16);
    long long nrun = (256 + units - 1) / units;
    if (nrun > N) nrun = N;
    vs->ncmax = ncmax;
    vs->nrun = (int)nrun;
    vs->plan_offset = (size_t)H * (size_t)ncmax * L.stride;
    vs->total = vs->plan_offset + 16 * (size_t)ncmax + 8 * ((size_t)N + 1) + 4 * ((size_t)nrun + 1);
    return KDA_OK;
}

int varlen_impl(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
                int chunk, const int *cu_seqlens, int N, int H, int T, int dk, int dv, int io, void *out,
                float *final_state, void *workspace, size_t workspace_bytes_given, hipStream_t stream,
                int gate_mode, unsigned long long *counts, const float *init_state) {
    VarlenSizes vs;
    int st = check_varlen(N, H, T, dk, dv, chunk, io, &vs);
    if (st != KDA_OK) return st;
    st = check_gate(g_min, gate_mode);
    if (st != KDA_OK) return st;
    if (!cu_seqlens || !workspace) return KDA_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !a || !beta || !out)) return KDA_ERR_NULL;  // empty arrays may be NULL
    const size_t esz = io == KDA_FP32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(a, 16) || !aligned(beta, esz) ||
        !aligned(out, 16) || !aligned(cu_seqlens, 4) || !aligned(workspace, 16) ||
        (final_state && !aligned(final_state, 16)) || (init_state && !aligned(init_state, 16)) ||
        (counts && !aligned(counts, 8)))
        return KDA_ERR_ALIGN;
    if (workspace_bytes_given < vs.total) return KDA_ERR_WORKSPACE;
    kda::LaunchArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
    p.g_min = g_min;
    p.logsig = gate_mode == KDA_GATE_LOGSIGMOID;
    p.chunk = chunk; p.B = 1; p.H = H; p.T = T; p.dk = dk; p.dv = dv;
    p.fp32 = io == KDA_FP32;
    p.out = out; p.final_state = final_state; p.init_state = init_state;
    p.workspace = workspace; p.counts = counts; p.stream = stream;
    p.cu = cu_seqlens; p.nseq = N; p.ncmax = (int)vs.ncmax; p.nrun = vs.nrun; p.plan_offset = vs.plan_offset;
    if (kda::launch_intra(p) != hipSuccess) return KDA_ERR_HIP;
    return kda::launch_state(p) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

// Backward: the 16-token chunk records, the chunk start states and the gradients of the chunk
// end states, in that order.
struct BwdSizes {
    size_t rec, states, total;
};

int check_bwd(int B, int H, int T, int dk, int dv, int io, BwdSizes *bs) {
    const int st = check_shape(B, H, T, dk, dv, 16, io);
    if (st != KDA_OK) return st;
    if ((long long)B * H > 65535) return KDA_ERR_SHAPE;  // grid y of the chunk-parallel gradient stage
    const KdaLayout L = kda_layout(16, dk, dv, io == KDA_FP32 ? 4 : 2);
    const size_t nch = (size_t)B * (size_t)H * (size_t)(T / 16);
    bs->rec = nch * L.stride;
    bs->states = nch * (size_t)dk * (size_t)dv * sizeof(float);
    bs->total = bs->rec + 2 * bs->states;
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char *kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "unsupported shape (dk, dv in {64,128}; B, H, N >= 1; T >= 0; T % chunk == 0 unless packed)";
    case KDA_ERR_DTYPE: return "io_dtype must be KDA_BF16 or KDA_FP32";
    case KDA_ERR_CHUNK: return "chunk must be 16, 32 or 64";
    case KDA_ERR_GMIN: return "g_min must be finite with KDA_G_MIN_LOWEST <= g_min < 0";
    case KDA_ERR_WORKSPACE: return "workspace missing or smaller than kda_chunk_fwd_workspace_bytes()";
    case KDA_ERR_HIP: return "a HIP call or kernel launch failed";
    case KDA_ERR_ALIGN: return "a pointer is not aligned as required (16 bytes; beta: element size)";
    case KDA_ERR_MODE: return "unknown gate_mode";
    case KDA_ERR_SCRATCH: return "problem needs more device scratch than KDA_NOALLOC_SCRATCH_BYTES (kda_chunk_fwd_noalloc)";
    default: return "unknown status";
    }
}

size_t kda_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int io_dtype) {
    if (check_shape(B, H, T, dk, dv, chunk, io_dtype) != KDA_OK) return 0;
    return workspace_bytes(B, H, T, dk, dv, chunk, io_dtype);
}

int kda_gate_cumsum(const void *a, float g_min, int chunk, int B, int H, int T, int dk, int io_dtype,
                    int gate_mode, float *G_out, hipStream_t stream) {
    int st = check_shape(B, H, T, dk, 64, chunk, io_dtype);
    if (st != KDA_OK) return st;
    st = check_gate(g_min, gate_mode);
    if (st != KDA_OK) return st;
    if (T > 0 && (!a || !G_out)) return KDA_ERR_NULL;  // empty arrays may be NULL
    if (!aligned(a, 16) || !aligned(G_out, 16)) return KDA_ERR_ALIGN;
    if (T == 0) return KDA_OK;
    kda::LaunchArgs p{};
    p.a = a; p.g_min = g_min; p.logsig = gate_mode == KDA_GATE_LOGSIGMOID;
    p.chunk = chunk; p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = 64;
    p.fp32 = io_dtype == KDA_FP32;
    p.G_out = G_out; p.stream = stream;
    return kda::launch_gate_cumsum(p) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_chunk_fwd(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
                  int chunk, int B, int H, int T, int dk, int dv, int io_dtype, void *out, float *final_state,
                  void *workspace, size_t workspace_bytes_given, hipStream_t stream) {
    return fwd_impl(q, k, v, a, beta, g_min, chunk, B, H, T, dk, dv, io_dtype, out, final_state, workspace,
                    workspace_bytes_given, stream, KDA_GATE_BOUNDED, nullptr, nullptr);
}

int kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const void *a, const void *beta,
                     float g_min, int chunk, int B, int H, int T, int dk, int dv, int io_dtype, void *out,
                     float *final_state, void *workspace, size_t workspace_bytes_given, hipStream_t stream,
                     int gate_mode, unsigned long long *nonfinite_counts, const float *initial_state) {
    return fwd_impl(q, k, v, a, beta, g_min, chunk, B, H, T, dk, dv, io_dtype, out, final_state, workspace,
                    workspace_bytes_given, stream, gate_mode, nonfinite_counts, initial_state);
}

int kda_chunk_intra(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
                    int chunk, int B, int H, int T, int dk, int dv, int io_dtype, void *workspace,
                    size_t workspace_bytes_given, hipStream_t stream, int gate_mode,
                    unsigned long long *nonfinite_counts) {
    return intra_impl(q, k, v, a, beta, g_min, chunk, B, H, T, dk, dv, io_dtype, workspace, workspace_bytes_given,
                      stream, gate_mode, nonfinite_counts, true);
}

int kda_chunk_state(const void *workspace, size_t workspace_bytes_given, int chunk, int B, int H, int T, int dk,
                    int dv, int io_dtype, void *out, float *final_state, hipStream_t stream,
                    unsigned long long *nonfinite_counts, const float *initial_state) {
    return state_impl(workspace, workspace_bytes_given, chunk, B, H, T, dk, dv, io_dtype, out, final_state, stream,
                      nonfinite_counts, initial_state, true);
}

int kda_chunk_fwd_lowrank(const void *q, const void *k, const void *v, const void *h, const void *z,
                          const float *A_log, const void *beta, float g_min, int chunk, int B, int H, int T, int dk,
                          int dv, int rank, int io_dtype, void *out, float *final_state, void *workspace,
                          size_t workspace_bytes_given, hipStream_t stream, int gate_mode,
                          unsigned long long *nonfinite_counts, const float *initial_state) {
    return fwd_impl(q, k, v, nullptr, beta, g_min, chunk, B, H, T, dk, dv, io_dtype, out, final_state, workspace,
                    workspace_bytes_given, stream, gate_mode, nonfinite_counts, initial_state,
                    LowRank{true, h, z, A_log, rank});
}

int kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *a, const void *beta,
                          float g_min, int chunk, int B, int H, int T, int dk, int dv, int io_dtype, void *out,
                          float *final_state, hipStream_t stream, int gate_mode, unsigned long long *nonfinite_counts,
                          const float *initial_state) {
    return noalloc_impl(q, k, v, a, beta, g_min, chunk, B, H, T, dk, dv, io_dtype, out, final_state, stream,
                        gate_mode, nonfinite_counts, initial_state);
}

size_t kda_chunk_fwd_varlen_workspace_bytes(int N, int H, int T, int dk, int dv, int chunk, int io_dtype) {
    VarlenSizes vs;
    if (check_varlen(N, H, T, dk, dv, chunk, io_dtype, &vs) != KDA_OK) return 0;
    return vs.total;
}

int kda_chunk_fwd_varlen(const void *q, const void *k, const void *v, const void *a, const void *beta,
                         float g_min, int chunk, const int *cu_seqlens, int N, int H, int T, int dk, int dv,
                         int io_dtype, void *out, float *final_state, void *workspace, size_t workspace_bytes_given,
                         hipStream_t stream, int gate_mode, unsigned long long *nonfinite_counts,
                         const float *initial_state) {
    return varlen_impl(q, k, v, a, beta, g_min, chunk, cu_seqlens, N, H, T, dk, dv, io_dtype, out, final_state,
                       workspace, workspace_bytes_given, stream, gate_mode, nonfinite_counts, initial_state);
}

size_t kda_chunk_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int io_dtype) {
    BwdSizes bs;
    if (check_bwd(B, H, T, dk, dv, io_dtype, &bs) != KDA_OK) return 0;
    return bs.total;
}

int kda_chunk_bwd(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min, int B,
                  int H, int T, int dk, int dv, int io_dtype, int gate_mode, const float *initial_state,
                  const void *dout, const float *dfinal_state, float *dq, float *dk_out, float *dv_out, float *da,
                  float *dbeta, float *dinitial_state, void *workspace, size_t workspace_bytes_given,
                  hipStream_t stream) {
    BwdSizes bs;
    int st = check_bwd(B, H, T, dk, dv, io_dtype, &bs);
    if (st != KDA_OK) return st;
    st = check_gate(g_min, gate_mode);
    if (st != KDA_OK) return st;
    if (T > 0 && (!q || !k || !v || !a || !beta || !dout || !dq || !dk_out || !dv_out || !da || !dbeta))
        return KDA_ERR_NULL;
    const size_t esz = io_dtype == KDA_FP32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(a, 16) || !aligned(beta, esz) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk_out, 16) || !aligned(dv_out, 16) || !aligned(da, 16) ||
        !aligned(dbeta, 4) || !aligned(initial_state, 16) || !aligned(dfinal_state, 16) ||
        !aligned(dinitial_state, 16) || !aligned(workspace, 16))
        return KDA_ERR_ALIGN;
    if (bs.total > 0 && (!workspace || workspace_bytes_given < bs.total)) return KDA_ERR_WORKSPACE;
    if (T == 0) {  // no tokens: the initial state's gradient is the final state's
        if (!dinitial_state) return KDA_OK;
        const size_t bytes = (size_t)B * H * dv * dk * sizeof(float);
        hipError_t e = dfinal_state
                           ? hipMemcpyAsync(dinitial_state, dfinal_state, bytes, hipMemcpyDeviceToDevice, stream)
                           : hipMemsetAsync(dinitial_state, 0, bytes, stream);
        return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    }
    kda::LaunchArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
    p.g_min = g_min;
    p.logsig = gate_mode == KDA_GATE_LOGSIGMOID;
    p.chunk = 16; p.B = B; p.H = H; p.T = T; p.dk = dk; p.dv = dv;
    p.fp32 = io_dtype == KDA_FP32;
    p.init_state = initial_state;
    p.workspace = workspace;
    p.states = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + bs.rec);
    p.dstates = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + bs.rec + bs.states);
    p.dout = dout; p.dfinal = dfinal_state;
    p.dq = dq; p.dk_ = dk_out; p.dv_ = dv_out; p.da = da; p.dbeta = dbeta; p.dinit = dinitial_state;
    p.stream = stream;
    return kda::launch_bwd(p) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step(const void *q, const void *k, const void *v, const void *a, const void *beta, float g_min,
                    int B, int H, int dk, int dv, int io_dtype, int gate_mode, float *state, void *out,
                    hipStream_t stream) {
    int st = check_shape(B, H, 16, dk, dv, 16, io_dtype);
    if (st != KDA_OK) return st;
    st = check_gate(g_min, gate_mode);
    if (st != KDA_OK) return st;
    if (!q || !k || !v || !a || !beta || !state || !out) return KDA_ERR_NULL;
    const size_t esz = io_dtype == KDA_FP32 ? 4 : 2;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(a, 16) || !aligned(beta, esz) ||
        !aligned(state, 16) || !aligned(out, 16))
        return KDA_ERR_ALIGN;
    kda::LaunchArgs p{};
    p.q = q; p.k = k; p.v = v; p.a = a; p.beta = beta;
    p.g_min = g_min;
    p.logsig = gate_mode == KDA_GATE_LOGSIGMOID;
    p.B = B; p.H = H; p.T = 1; p.dk = dk; p.dv = dv;
    p.fp32 = io_dtype == KDA_FP32;
    p.state = state; p.out = out; p.stream = stream;
    return kda::launch_decode(p) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
