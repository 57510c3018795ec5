"""Parity of the packed-documents forward (kda_chunk_fwd_varlen, through the C ABI)
with the float64 oracle, same bar as the chunked forward: bf16 I/O max|d| <=
2e-2 RMS + u_bf16 |ref| element-wise, fp32 I/O <= 1e-4 absolute, final states
per document against the RMS of the oracle's states.

Cases: length mixes around the chunk size (1, C-1, C, C+1, empty documents, a
stream length that is not a multiple of the chunk) for every chunk size and
head-dimension pair, with and without initial states; documents that are all
whole chunks against the fixed-length path (bit for bit); boundaries with runs
of empty documents and one document covering the stream; the 64k packed
workload at full size in the benchmark's launch configuration, with every
output and final state of sampled documents checked.
"""
import numpy as np
import pytest
import torch

import chunked_gated_linear_bounded_amd as kda
import kda_inputs as KI
from oracle import native
from parity_util import _say, _tol_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.lib()


def _packed_case(lengths, io, seed, dk=128, dv=128, chunk=64, H=2, a_sigma=4.0):
    T = int(sum(lengths))
    w = KI.Workload("p%d" % seed, 1, H, T, dk, dv, chunk, io, a_sigma, False, seed)
    inp = KI.make_packed_inputs(w)
    cu = KI.cu_seqlens(lengths)
    return w, {n: t.cuda() for n, t in inp.items()}, cu


def _f64(inp):
    return {n: t.double().cpu().numpy() for n, t in inp.items()}


def _states(N, w, seed):
    rng = np.random.default_rng(2000 + seed)
    return torch.from_numpy((rng.standard_normal((N, w.H, w.dv, w.dk)) * 0.5).astype(np.float32)).cuda()


CASES = [
    ("fp32", 16, 64, 64, [1, 15, 16, 17, 40, 0, 33]),
    ("fp32", 32, 128, 64, [31, 32, 33, 0, 0, 5, 64]),
    ("fp32", 64, 64, 128, [64, 1, 63, 65, 130]),
    ("bf16", 16, 128, 128, [3, 16, 0, 29, 48, 1]),
    ("bf16", 32, 64, 128, [100, 1, 31, 33, 64]),
    ("bf16", 64, 128, 128, [1, 63, 64, 65, 200, 0, 130, 7]),
    ("bf16", 64, 128, 64, [250, 6]),
]


@pytest.mark.parametrize("with_s0", [False, True])
@pytest.mark.parametrize("io,chunk,dk,dv,lengths", CASES)
def test_packed_parity(io, chunk, dk, dv, lengths, with_s0):
    seed = 61 + len(lengths) + chunk
    w, inp, cu = _packed_case(lengths, io, seed, dk=dk, dv=dv, chunk=chunk)
    N = len(lengths)
    S0 = _states(N, w, seed) if with_s0 else None
    _say(io, chunk, dk, dv, lengths, "s0" if with_s0 else "")
    out, fs = kda.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                   torch.from_numpy(cu).cuda(), chunk=chunk, return_final_state=True,
                                   initial_state=S0)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent_varlen(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], cu,
                                     S0=None if S0 is None else S0.double().cpu().numpy())
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(fs.double().cpu().numpy(), rf, io, "final_state")


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("fp32", 16)])
def test_whole_chunk_documents_match_the_batched_path(io, chunk):
    """N documents of equal length L (a multiple of the chunk) packed into one stream give
    bit for bit what the fixed-length path gives for a batch of N sequences of length L."""
    N, L, H = 3, 4 * chunk, 2
    w = KI.Workload("b", N, H, L, 128, 128, chunk, io, 4.0, False, 71)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    S0 = torch.randn(N, H, 128, 128, device="cuda") * 0.5
    ob, fb = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], chunk=chunk,
                           return_final_state=True, initial_state=S0)
    pk = {n: t.transpose(0, 1).reshape(H, N * L, *t.shape[3:]).contiguous() for n, t in inp.items()}
    cu = torch.from_numpy(KI.cu_seqlens([L] * N)).cuda()
    op, fp = kda.chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["a"], pk["beta"], cu, chunk=chunk,
                                  return_final_state=True, initial_state=S0)
    torch.cuda.synchronize()
    assert torch.equal(op, ob.transpose(0, 1).reshape(H, N * L, -1))
    assert torch.equal(fp, fb)


def test_runs_of_empty_documents_and_one_covering_document():
    lengths = [0, 0, 300, 0, 0, 0]
    w, inp, cu = _packed_case(lengths, "bf16", 72, dk=64, dv=64)
    N = len(lengths)
    S0 = _states(N, w, 72)
    out, fs = kda.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                   torch.from_numpy(cu).cuda(), return_final_state=True, initial_state=S0)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent_varlen(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], cu,
                                     S0=S0.double().cpu().numpy())
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")
    for i in (0, 1, 3, 4, 5):  # empty documents: the initial state passes through unchanged
        assert torch.equal(fs[i], S0[i])


def test_thousands_of_short_documents():
    """2,600 documents of 0 to 40 tokens (about one in ten empty): the plan kernel's scans run
    over three 1024-document tiles and the chunk table holds thousands of short chunks; every
    output and every document's final state against the oracle."""
    rng = np.random.default_rng(74)
    lengths = [int(x) if rng.random() > 0.1 else 0 for x in rng.integers(1, 41, size=2600)]
    w, inp, cu = _packed_case(lengths, "bf16", 74, dk=64, dv=64, chunk=16, H=3)
    N = len(lengths)
    S0 = _states(N, w, 74)
    _say("documents", N, "tokens", w.T)
    out, fs = kda.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                   torch.from_numpy(cu).cuda(), chunk=16, return_final_state=True, initial_state=S0)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent_varlen(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], cu,
                                     S0=S0.double().cpu().numpy())
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")
    for i in range(N):
        if lengths[i] == 0:  # an empty document keeps its initial state exactly
            assert torch.equal(fs[i], S0[i])


def test_in_place_states():
    """initial_state and final_state may be one array (each document's state is read before it is
    written)."""
    lengths = [70, 5, 129]
    w, inp, cu = _packed_case(lengths, "bf16", 73)
    S0 = _states(3, w, 73)
    S = S0.clone()
    out = kda.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], torch.from_numpy(cu).cuda(),
                               final_state=S, initial_state=S)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent_varlen(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], cu,
                                     S0=S0.double().cpu().numpy())
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(S.double().cpu().numpy(), rf, "bf16", "final_state")


def test_packed_64k_workload_sampled_documents():
    """The 64k packed stream (32 heads, documents log-uniform in [32, 4096] tokens) at full size,
    launched as the benchmark launches it; every output and the final state of four documents
    (the first, the last, the longest and a short one) on three heads against the oracle, and no
    non-finite operand or output anywhere."""
    w = KI.PACKED
    lengths = KI.packed_lengths(w.T, w.seed)
    cu = KI.cu_seqlens(lengths)
    _say("packed64k:", len(lengths), "documents, generating on GPU")
    inp = KI.make_packed_inputs(w, device="cuda")
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, fs = kda.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"],
                                   torch.from_numpy(cu).cuda(), chunk=w.chunk, return_final_state=True,
                                   counts=counts)
    torch.cuda.synchronize()
    assert counts.tolist() == [0, 0]
    short = min(range(len(lengths)), key=lambda i: lengths[i])
    docs = sorted({0, len(lengths) - 1, int(np.argmax(lengths)), short})
    for h in (0, 17, 31):
        for i in docs:
            s, e = int(cu[i]), int(cu[i + 1])
            _say(" head", h, "document", i, "tokens", s, e)
            sl = {n: t[h:h + 1, s:e].double().cpu().numpy() for n, t in inp.items()}
            ro, rf = native.recurrent_varlen(sl["q"], sl["k"], sl["v"], sl["a"], sl["beta"], [0, e - s])
            _tol_check(out[h, s:e].double().cpu().numpy(), ro[0], w.io)
            _tol_check(fs[i, h].double().cpu().numpy(), rf[0, 0], w.io, "final_state")
