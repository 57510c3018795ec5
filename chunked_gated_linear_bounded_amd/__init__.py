"""MI355X (gfx950) chunked forward of bounded-decay KDA -- Python binding.

A thin ctypes layer over libkda.so (include/kda.h).  It only marshals
arguments: torch supplies device memory and the current HIP stream, every step
of the computation runs in the library's HIP kernels.  If the library is not
built, every entry point raises; there is no fallback.

    import chunked_gated_linear_bounded_amd as kda
    out, S = kda.chunk_fwd(q, k, v, a, beta, g_min=-5.0, chunk=64, return_final_state=True)
    out2 = kda.chunk_fwd(q2, k2, v2, a2, beta2, initial_state=S)     # continue the sequence
    o_t = kda.decode_step(q_t, k_t, v_t, a_t, beta_t, S)               # one more token, S in place
    o = kda.chunk_fwd_varlen(q, k, v, a, beta, cu_seqlens)             # packed documents, [H,T,d]
    o = kda.chunk_fwd_lowrank(q, k, v, h, z, A_log, beta)              # a = e^A (h z^T) in-kernel
    g = kda.chunk_bwd(q, k, v, a, beta, dout)                          # gradients (training)
    out, S = kda.KdaChunkFunction.apply(q, k, v, a, beta)              # the same, under autograd
    G = kda.gate_cumsum(a, g_min=-5.0, chunk=64)
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
KDA_BF16, KDA_FP32 = 0, 1
GATE_MODES = {"bounded": 0, "logsigmoid": 1}
_DTYPES = {torch.bfloat16: KDA_BF16, torch.float32: KDA_FP32}

_lib = None


class KdaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %d (%s)" % (fn, status, status_string(status)))


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libkda.so not built: run python -m chunked_gated_linear_bounded_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.kda_abi_version.restype = i
        L.kda_status_string.argtypes = [i]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_chunk_fwd_workspace_bytes.argtypes = [i] * 7
        L.kda_chunk_fwd_workspace_bytes.restype = sz
        L.kda_gate_cumsum.argtypes = [vp, f, i, i, i, i, i, i, i, vp, vp]
        L.kda_gate_cumsum.restype = i
        L.kda_chunk_fwd.argtypes = [vp] * 5 + [f] + [i] * 7 + [vp, vp, vp, sz, vp]
        L.kda_chunk_fwd.restype = i
        L.kda_chunk_fwd_ex.argtypes = [vp] * 5 + [f] + [i] * 7 + [vp, vp, vp, sz, vp, i, vp, vp]
        L.kda_chunk_fwd_ex.restype = i
        L.kda_chunk_intra.argtypes = [vp] * 5 + [f] + [i] * 7 + [vp, sz, vp, i, vp]
        L.kda_chunk_intra.restype = i
        L.kda_chunk_state.argtypes = [vp, sz] + [i] * 7 + [vp, vp, vp, vp, vp]
        L.kda_chunk_state.restype = i
        L.kda_chunk_fwd_lowrank.argtypes = [vp] * 7 + [f] + [i] * 8 + [vp, vp, vp, sz, vp, i, vp, vp]
        L.kda_chunk_fwd_lowrank.restype = i
        L.kda_chunk_fwd_varlen_workspace_bytes.argtypes = [i] * 7
        L.kda_chunk_fwd_varlen_workspace_bytes.restype = sz
        L.kda_chunk_fwd_varlen.argtypes = [vp] * 5 + [f, i, vp] + [i] * 6 + [vp, vp, vp, sz, vp, i, vp, vp]
        L.kda_chunk_fwd_varlen.restype = i
        L.kda_chunk_bwd_workspace_bytes.argtypes = [i] * 6
        L.kda_chunk_bwd_workspace_bytes.restype = sz
        L.kda_chunk_bwd.argtypes = [vp] * 5 + [f] + [i] * 7 + [vp] * 10 + [sz, vp]
        L.kda_chunk_bwd.restype = i
        L.kda_decode_step.argtypes = [vp] * 5 + [f] + [i] * 6 + [vp, vp, vp]
        L.kda_decode_step.restype = i
        L.kda_chunk_fwd_noalloc.argtypes = [vp] * 5 + [f] + [i] * 7 + [vp, vp, vp, i, vp, vp]
        L.kda_chunk_fwd_noalloc.restype = i
        _lib = L
    return _lib


def abi_version() -> int:
    return int(lib().kda_abi_version())


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def workspace_bytes(B, H, T, dk, dv, chunk, dtype) -> int:
    io = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().kda_chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, io))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A new tensor for the library to write on `stream` (None: the current stream).  The caching
    allocator ties a block to the stream it was allocated on and hands it out again, once freed,
    only to work on that stream; allocating on the launch stream keeps a block that the caller
    drops before the kernels finish (the workspace, always) from going to other work meanwhile."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _check(t, name, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def gate_cumsum(a, g_min=-5.0, chunk=64, gate="bounded", out=None, stream=None):
    """G[b,h,t,c] = sum of g over t's chunk up to t (natural log), float32."""
    _check(a, "a")
    B, H, T, dk = a.shape
    if out is None:
        out = _empty((B, H, T, dk), torch.float32, a.device, stream)
    _check(out, "out", torch.float32, a.device)
    st = lib().kda_gate_cumsum(_ptr(a), float(g_min), int(chunk), B, H, T, dk, _DTYPES[a.dtype],
                               GATE_MODES[gate], _ptr(out), _stream(stream))
    if st != KDA_OK:
        raise KdaError("kda_gate_cumsum", st)
    return out


def chunk_fwd(q, k, v, a, beta, g_min=-5.0, chunk=64, out=None, final_state=None,
              return_final_state=False, workspace=None, stream=None, gate="bounded", counts=None,
              initial_state=None):
    """Chunked KDA forward.  q, k, a: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T];
    all bf16 or all float32, contiguous, on one GPU.  Returns out [B,H,T,dv]
    (and the float32 final state [B,H,dv,dk] when asked for).  `counts`: optional
    int64 GPU tensor of 2 elements that non-finite counters are added to.
    `initial_state`: optional float32 [B,H,dv,dk] state to start from (may be
    passed as final_state too, to continue in place)."""
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (a, "a"), (beta, "beta")):
        _check(t, n, dtype, dev)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or a.shape != q.shape or v.shape != (B, H, T, dv) or beta.shape != (B, H, T):
        raise ValueError("shape mismatch")
    if out is None:
        out = _empty((B, H, T, dv), dtype, dev, stream)
    _check(out, "out", dtype, dev)
    if final_state is None and return_final_state:
        final_state = _empty((B, H, dv, dk), torch.float32, dev, stream)
    if final_state is not None:
        _check(final_state, "final_state", torch.float32, dev)
    need = workspace_bytes(B, H, T, dk, dv, chunk, dtype)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, dev, stream)
    _check(workspace, "workspace", torch.uint8, dev)
    if counts is not None:
        _check(counts, "counts", torch.int64, dev)
    if initial_state is not None:
        _check(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (B, H, dv, dk):
            raise ValueError("initial_state must be [B,H,dv,dk]")
    L = lib()
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), float(g_min), int(chunk), B, H, T, dk, dv,
            _DTYPES[dtype], _ptr(out), _ptr(final_state), _ptr(workspace), workspace.numel(), _stream(stream)]
    if gate == "bounded" and counts is None and initial_state is None:
        st = L.kda_chunk_fwd(*args)
        fn = "kda_chunk_fwd"
    else:
        st = L.kda_chunk_fwd_ex(*args, GATE_MODES[gate], _ptr(counts), _ptr(initial_state))
        fn = "kda_chunk_fwd_ex"
    if st != KDA_OK:
        raise KdaError(fn, st)
    if return_final_state:
        return out, final_state
    return out


def chunk_fwd_noalloc(q, k, v, a, beta, out, g_min=-5.0, chunk=64, final_state=None, stream=None,
                      gate="bounded", counts=None, initial_state=None):
    """chunk_fwd through kda_chunk_fwd_noalloc, which allocates no device memory (its chunk records
    live in a static device array of the library): for callers that cannot allocate, such as code
    under graph capture.  out [B,H,T,dv] (and final_state [B,H,dv,dk] float32, if wanted) must be
    given; nothing is allocated here either.  Calls on one GPU share that array, so they must not
    overlap in time."""
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (a, "a"), (beta, "beta")):
        _check(t, n, dtype, dev)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or a.shape != q.shape or v.shape != (B, H, T, dv) or beta.shape != (B, H, T) or \
            tuple(out.shape) != (B, H, T, dv):
        raise ValueError("shape mismatch")
    _check(out, "out", dtype, dev)
    for t, n in ((final_state, "final_state"), (initial_state, "initial_state")):
        if t is not None:
            _check(t, n, torch.float32, dev)
            if tuple(t.shape) != (B, H, dv, dk):
                raise ValueError("%s must be [B,H,dv,dk]" % n)
    if counts is not None:
        _check(counts, "counts", torch.int64, dev)
    st = lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), float(g_min), int(chunk), B, H,
                                     T, dk, dv, _DTYPES[dtype], _ptr(out), _ptr(final_state), _stream(stream),
                                     GATE_MODES[gate], _ptr(counts), _ptr(initial_state))
    if st != KDA_OK:
        raise KdaError("kda_chunk_fwd_noalloc", st)
    return out


def chunk_intra(q, k, v, a, beta, workspace, g_min=-5.0, chunk=64, stream=None, gate="bounded", counts=None):
    """First stage of chunk_fwd: fills `workspace` (uint8 GPU tensor of at least
    workspace_bytes(...) bytes) with the per-chunk operands."""
    dtype, dev = q.dtype, q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (a, "a"), (beta, "beta")):
        _check(t, n, dtype, dev)
    _check(workspace, "workspace", torch.uint8, dev)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    st = lib().kda_chunk_intra(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), float(g_min), int(chunk), B, H, T,
                               dk, dv, _DTYPES[dtype], _ptr(workspace), workspace.numel(), _stream(stream),
                               GATE_MODES[gate], _ptr(counts))
    if st != KDA_OK:
        raise KdaError("kda_chunk_intra", st)


def chunk_state(workspace, out, final_state=None, chunk=64, dk=None, stream=None, counts=None,
                initial_state=None):
    """Second stage of chunk_fwd: reads `workspace`, writes out [B,H,T,dv] (and
    final_state [B,H,dv,dk] float32 when given), starting from initial_state
    when given.  dk defaults to dv."""
    _check(out, "out")
    _check(workspace, "workspace", torch.uint8, out.device)
    B, H, T, dv = out.shape
    dk = dv if dk is None else dk
    st = lib().kda_chunk_state(_ptr(workspace), workspace.numel(), int(chunk), B, H, T, dk, dv, _DTYPES[out.dtype],
                               _ptr(out), _ptr(final_state), _stream(stream), _ptr(counts), _ptr(initial_state))
    if st != KDA_OK:
        raise KdaError("kda_chunk_state", st)


def chunk_fwd_lowrank(q, k, v, h, z, A_log, beta, g_min=-5.0, chunk=64, out=None, final_state=None,
                      return_final_state=False, initial_state=None, workspace=None, stream=None, gate="bounded",
                      counts=None):
    """Chunked forward with the gate pre-activation a = exp(A_log) * (h z^T) formed in the chunk
    kernel: h [B,T,R] (shared by the heads), z [H,dk,R] in the I/O dtype, A_log [H,dk] float32;
    q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T].  Otherwise as chunk_fwd."""
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (h, "h"), (z, "z"), (beta, "beta")):
        _check(t, n, dtype, dev)
    _check(A_log, "A_log", torch.float32, dev)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    R = h.shape[-1]
    if k.shape != q.shape or v.shape != (B, H, T, dv) or beta.shape != (B, H, T) or h.shape != (B, T, R) or \
            z.shape != (H, dk, R) or A_log.shape != (H, dk):
        raise ValueError("shape mismatch")
    if out is None:
        out = _empty((B, H, T, dv), dtype, dev, stream)
    _check(out, "out", dtype, dev)
    if final_state is None and return_final_state:
        final_state = _empty((B, H, dv, dk), torch.float32, dev, stream)
    for t, n in ((final_state, "final_state"), (initial_state, "initial_state")):
        if t is not None:
            _check(t, n, torch.float32, dev)
            if tuple(t.shape) != (B, H, dv, dk):
                raise ValueError("%s must be [B,H,dv,dk]" % n)
    need = workspace_bytes(B, H, T, dk, dv, chunk, dtype)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, dev, stream)
    _check(workspace, "workspace", torch.uint8, dev)
    if counts is not None:
        _check(counts, "counts", torch.int64, dev)
    st = lib().kda_chunk_fwd_lowrank(_ptr(q), _ptr(k), _ptr(v), _ptr(h), _ptr(z), _ptr(A_log), _ptr(beta),
                                     float(g_min), int(chunk), B, H, T, dk, dv, R, _DTYPES[dtype], _ptr(out),
                                     _ptr(final_state), _ptr(workspace), workspace.numel(), _stream(stream),
                                     GATE_MODES[gate], _ptr(counts), _ptr(initial_state))
    if st != KDA_OK:
        raise KdaError("kda_chunk_fwd_lowrank", st)
    if return_final_state:
        return out, final_state
    return out


def varlen_workspace_bytes(N, H, T, dk, dv, chunk, dtype) -> int:
    io = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().kda_chunk_fwd_varlen_workspace_bytes(N, H, T, dk, dv, chunk, io))


def chunk_fwd_varlen(q, k, v, a, beta, cu_seqlens, g_min=-5.0, chunk=64, out=None, final_state=None,
                     return_final_state=False, initial_state=None, workspace=None, stream=None, gate="bounded",
                     counts=None):
    """Packed documents: q, k, a [H,T,dk]; v [H,T,dv]; beta [H,T] (all bf16 or all float32);
    cu_seqlens int32 GPU tensor [N+1] of document boundaries (0 ... T).  Each document
    runs from its own state: initial_state / final_state are float32 [N,H,dv,dk].
    Returns out [H,T,dv] (and the final states when asked for)."""
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (a, "a"), (beta, "beta")):
        _check(t, n, dtype, dev)
    _check(cu_seqlens, "cu_seqlens", torch.int32, dev)
    H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or a.shape != q.shape or v.shape != (H, T, dv) or beta.shape != (H, T) or \
            cu_seqlens.dim() != 1:
        raise ValueError("shape mismatch")
    N = cu_seqlens.numel() - 1
    if out is None:
        out = _empty((H, T, dv), dtype, dev, stream)
    _check(out, "out", dtype, dev)
    if final_state is None and return_final_state:
        final_state = _empty((N, H, dv, dk), torch.float32, dev, stream)
    for t, n in ((final_state, "final_state"), (initial_state, "initial_state")):
        if t is not None:
            _check(t, n, torch.float32, dev)
            if tuple(t.shape) != (N, H, dv, dk):
                raise ValueError("%s must be [N,H,dv,dk]" % n)
    need = varlen_workspace_bytes(N, H, T, dk, dv, chunk, dtype)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, dev, stream)
    _check(workspace, "workspace", torch.uint8, dev)
    if counts is not None:
        _check(counts, "counts", torch.int64, dev)
    st = lib().kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), float(g_min), int(chunk),
                                    _ptr(cu_seqlens), N, H, T, dk, dv, _DTYPES[dtype], _ptr(out), _ptr(final_state),
                                    _ptr(workspace), workspace.numel(), _stream(stream), GATE_MODES[gate],
                                    _ptr(counts), _ptr(initial_state))
    if st != KDA_OK:
        raise KdaError("kda_chunk_fwd_varlen", st)
    if return_final_state:
        return out, final_state
    return out


def bwd_workspace_bytes(B, H, T, dk, dv, dtype) -> int:
    io = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return int(lib().kda_chunk_bwd_workspace_bytes(B, H, T, dk, dv, io))


def chunk_bwd(q, k, v, a, beta, dout, g_min=-5.0, initial_state=None, dfinal_state=None, gate="bounded",
              workspace=None, stream=None, want_dinitial=True):
    """Gradients of sum(dout * out) + sum(dfinal_state * final_state) of chunk_fwd with respect to
    q, k, v, a, beta and the initial state.  Inputs as chunk_fwd (T % 16 == 0), dout [B,H,T,dv] in
    the I/O dtype, dfinal_state float32 [B,H,dv,dk] or None.  Returns a dict of float32 tensors
    dq, dk, dv, da, dbeta and dinitial_state (None unless want_dinitial)."""
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (a, "a"), (beta, "beta"), (dout, "dout")):
        _check(t, n, dtype, dev)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or a.shape != q.shape or v.shape != (B, H, T, dv) or beta.shape != (B, H, T) or \
            dout.shape != v.shape:
        raise ValueError("shape mismatch")
    for t, n in ((initial_state, "initial_state"), (dfinal_state, "dfinal_state")):
        if t is not None:
            _check(t, n, torch.float32, dev)
            if tuple(t.shape) != (B, H, dv, dk):
                raise ValueError("%s must be [B,H,dv,dk]" % n)
    def f32(*shape):
        return _empty(shape, torch.float32, dev, stream)

    g = {"dq": f32(B, H, T, dk), "dk": f32(B, H, T, dk), "dv": f32(B, H, T, dv), "da": f32(B, H, T, dk),
         "dbeta": f32(B, H, T), "dinitial_state": f32(B, H, dv, dk) if want_dinitial else None}
    need = bwd_workspace_bytes(B, H, T, dk, dv, dtype)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, dev, stream)
    _check(workspace, "workspace", torch.uint8, dev)
    st = lib().kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), float(g_min), B, H, T, dk, dv,
                             _DTYPES[dtype], GATE_MODES[gate], _ptr(initial_state), _ptr(dout), _ptr(dfinal_state),
                             _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["da"]), _ptr(g["dbeta"]),
                             _ptr(g["dinitial_state"]), _ptr(workspace), workspace.numel(), _stream(stream))
    if st != KDA_OK:
        raise KdaError("kda_chunk_bwd", st)
    return g


class KdaChunkFunction(torch.autograd.Function):
    """out, final_state = KdaChunkFunction.apply(q, k, v, a, beta, g_min, chunk, gate): the chunked
    forward with its backward, for training.  Forward through kda_chunk_fwd_ex, backward through
    kda_chunk_bwd (T % 16 == 0); the float32 gradients are returned in the inputs' dtype.  No
    initial state (S_0 = 0)."""

    @staticmethod
    def forward(ctx, q, k, v, a, beta, g_min=-5.0, chunk=64, gate="bounded"):
        out, fs = chunk_fwd(q, k, v, a, beta, g_min=g_min, chunk=chunk, return_final_state=True, gate=gate)
        ctx.save_for_backward(q, k, v, a, beta)
        ctx.g_min, ctx.gate = g_min, gate
        return out, fs

    @staticmethod
    def backward(ctx, dout, dfinal):
        q, k, v, a, beta = ctx.saved_tensors
        dout = torch.zeros_like(q[..., :1].expand(*q.shape[:-1], v.shape[-1])) if dout is None else dout
        g = chunk_bwd(q, k, v, a, beta, dout.contiguous().to(q.dtype), ctx.g_min,
                      dfinal_state=None if dfinal is None else dfinal.contiguous().float(), gate=ctx.gate,
                      want_dinitial=False)
        return (g["dq"].to(q.dtype), g["dk"].to(k.dtype), g["dv"].to(v.dtype), g["da"].to(a.dtype),
                g["dbeta"].to(beta.dtype), None, None, None)


def decode_step(q, k, v, a, beta, state, g_min=-5.0, gate="bounded", out=None, stream=None):
    """One token per (batch, head): q, k, a [B,H,dk]; v [B,H,dv]; beta [B,H] (all bf16
    or all float32); state float32 [B,H,dv,dk], updated in place.  Returns out [B,H,dv]."""
    dtype = q.dtype
    if dtype not in _DTYPES:
        raise ValueError("unsupported dtype %s" % dtype)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (a, "a"), (beta, "beta")):
        _check(t, n, dtype, dev)
    _check(state, "state", torch.float32, dev)
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or a.shape != q.shape or v.shape != (B, H, dv) or beta.shape != (B, H) or \
            tuple(state.shape) != (B, H, dv, dk):
        raise ValueError("shape mismatch")
    if out is None:
        out = _empty((B, H, dv), dtype, dev, stream)
    _check(out, "out", dtype, dev)
    st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(beta), float(g_min), B, H, dk, dv,
                               _DTYPES[dtype], GATE_MODES[gate], _ptr(state), _ptr(out), _stream(stream))
    if st != KDA_OK:
        raise KdaError("kda_decode_step", st)
    return out
