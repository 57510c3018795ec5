"""The allocation-free forward, kda_chunk_fwd_noalloc, against kda_chunk_fwd_ex on the same inputs.

kda_chunk_fwd_noalloc runs the sequence in windows of chunks whose records fit its static device
scratch, carrying the state from window to window; its outputs and final state must agree with the
allocating entry point's to the parity bar (tests/parity_util.py), with those as the reference.
Two calls in a row on one GPU, the second smaller: a long 32-head sequence over several windows
with the state carried in final_state, then a short one from an initial state with no final_state
(the state then carried in the scratch itself).
"""
import numpy as np
import pytest
import torch

import chunked_gated_linear_bounded_amd as kda
import kda_inputs as KI
from parity_util import _say, _tol_check

pytestmark = pytest.mark.gpu

SCRATCH = 128 << 20


def _ref(inp, chunk, init=None, gate="bounded"):
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], chunk=chunk, return_final_state=True,
                            initial_state=init, gate=gate, counts=counts)
    return out, fs, counts


def _windows(w):
    rec = kda.workspace_bytes(1, 1, w.chunk, w.dk, w.dv, w.chunk, w.torch_dtype)
    return -(-(w.T // w.chunk) // (SCRATCH // (w.B * w.H * rec)))


def test_noalloc_matches_the_allocating_forward_twice():
    assert torch.cuda.is_available()
    # call 1: B=1, H=32, T=8192, bf16, chunk 64 -- three windows of at most 50 chunks
    w1 = KI.Workload("na1", 1, 32, 8192, 128, 128, 64, "bf16", 4.0, False, 801)
    _say("noalloc call 1:", w1, "windows", _windows(w1))
    assert _windows(w1) >= 3
    inp = KI.make_inputs(w1, device="cuda")
    ro, rf, rc = _ref(inp, w1.chunk)
    out = torch.full_like(ro, float("nan"))
    fs = torch.full_like(rf, float("nan"))
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=w1.chunk, final_state=fs,
                          counts=counts)
    torch.cuda.synchronize()
    assert counts.tolist() == rc.tolist() == [0, 0]
    _tol_check(out.double().cpu().numpy(), ro.double().cpu().numpy(), "bf16", "out (call 1)")
    _tol_check(fs.double().cpu().numpy(), rf.double().cpu().numpy(), "bf16", "final_state (call 1)")
    del inp, ro, rf, out, fs
    # call 2, smaller: B=2, H=3, T=640, fp32, chunk 32, from an initial state, no final_state
    w2 = KI.Workload("na2", 2, 3, 640, 64, 128, 32, "fp32", 2.0, False, 802)
    _say("noalloc call 2:", w2)
    inp = KI.make_inputs(w2, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(803)
    init = 0.3 * torch.randn((w2.B, w2.H, w2.dv, w2.dk), generator=gen, device="cuda")
    ro, _, _ = _ref(inp, w2.chunk, init)
    out = torch.full_like(ro, float("nan"))
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=w2.chunk,
                          initial_state=init)
    torch.cuda.synchronize()
    _tol_check(out.double().cpu().numpy(), ro.double().cpu().numpy(), "fp32", "out (call 2)")


def test_noalloc_windows_with_the_state_in_the_scratch():
    # a sequence of several windows with no final_state: the state crosses window boundaries through
    # the scratch; then the same call with the unbounded gate counts what the allocating one counts
    w = KI.Workload("na3", 2, 16, 4096, 128, 128, 64, "bf16", 4.0, False, 804)
    _say("noalloc, state in the scratch:", w, "windows", _windows(w))
    assert _windows(w) >= 2
    inp = KI.make_inputs(w, device="cuda")
    ro, _, _ = _ref(inp, w.chunk)
    out = torch.full_like(ro, float("nan"))
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=w.chunk)
    torch.cuda.synchronize()
    _tol_check(out.double().cpu().numpy(), ro.double().cpu().numpy(), "bf16", "out")
    inp["a"] = torch.where(inp["a"].float() < -2.0, -40.0, inp["a"].float()).to(inp["a"].dtype)
    _, _, rc = _ref(inp, w.chunk, gate="logsigmoid")
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=w.chunk, gate="logsigmoid",
                          counts=counts)
    torch.cuda.synchronize()
    _say("  unbounded gate counts: noalloc", counts.tolist(), "allocating", rc.tolist())
    assert rc.tolist()[0] > 0 and counts.tolist()[0] == rc.tolist()[0]


def test_noalloc_empty_sequence_and_the_size_limit():
    # T = 0: final_state receives the initial state (written by a kernel, no memset or copy)
    inp = {n: torch.empty((1, 2, 0, 64) if n != "beta" else (1, 2, 0), dtype=torch.bfloat16, device="cuda")
           for n in ("q", "k", "v", "a", "beta")}
    init = torch.randn((1, 2, 64, 64), device="cuda")
    fs = torch.full_like(init, float("nan"))
    out = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=16, final_state=fs,
                          initial_state=init)
    fs0 = torch.full_like(init, float("nan"))
    kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=16, final_state=fs0)
    torch.cuda.synchronize()
    assert torch.equal(fs, init) and torch.count_nonzero(fs0).item() == 0
    # more heads than one chunk of each fits: rejected before anything runs
    H = 2048
    x = torch.zeros((1, H, 64, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((1, H, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kda.KdaError) as ei:
        kda.chunk_fwd_noalloc(x, x, x, x, b, torch.empty_like(x), chunk=64, final_state=None)
    assert ei.value.status == -10
    _say("  rejected:", ei.value)
    np.testing.assert_equal(torch.count_nonzero(x).item(), 0)
