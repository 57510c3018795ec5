"""Parity of the backward pass (kda_chunk_bwd, through the C ABI) with the float64 oracle's
hand-written adjoint (oracle.native.backward, itself pinned by finite differences): every
gradient (q, k, v, a, beta, initial state) for an objective sum(dout * out) +
sum(dfinal * final_state).  Gradients are float32; bar per element: bf16 inputs
2e-2 RMS + u_bf16 |ref|, fp32 inputs 1e-4 max(1, RMS).

Cases: every head-dimension pair and both I/O types over several 16-token chunks, with and
without an initial state and a final-state gradient; the unbounded gate; a batch; a
2048-token sequence in full; the 64k workload (H=32, T=65536, d=128, bf16) at full size, two
heads checked over all their tokens.
"""
import numpy as np
import pytest
import torch

import chunked_gated_linear_bounded_amd as kda
import kda_inputs as KI
from oracle import native
from parity_util import _grad_check, _say

pytestmark = pytest.mark.gpu

KEYS = (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("da", "da"), ("dbeta", "dbeta"), ("dinitial_state", "dS0"))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.lib()


def _run_and_check(w, inp, dout, S0, dF, gate="bounded", heads=None):
    g = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], dout, initial_state=S0,
                      dfinal_state=dF, gate=gate)
    torch.cuda.synchronize()
    hs = range(w.H) if heads is None else heads
    for h in hs:
        x = {n: t[:, h:h + 1].double().cpu().numpy() for n, t in inp.items()}
        ref = native.backward(x["q"], x["k"], x["v"], x["a"], x["beta"], dout[:, h:h + 1].double().cpu().numpy(),
                              -5.0, gate, S0=None if S0 is None else S0[:, h:h + 1].double().cpu().numpy(),
                              dfinal=None if dF is None else dF[:, h:h + 1].double().cpu().numpy())
        for key, rkey in KEYS:
            _grad_check(g[key][:, h:h + 1].double().cpu().numpy(), ref[rkey], w.io, "%s head %d" % (key, h))


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("io,dk,dv", [("fp32", 64, 64), ("fp32", 128, 64), ("fp32", 64, 128), ("fp32", 128, 128),
                                      ("bf16", 64, 64), ("bf16", 128, 64), ("bf16", 64, 128), ("bf16", 128, 128)])
def test_bwd_small(io, dk, dv, with_state):
    w = KI.Workload("bw", 1, 2, 80, dk, dv, 16, io, 2.0, False, 101 + dk + dv)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout, dF = (t.cuda() for t in KI.make_grads(w))
    S0 = torch.randn(1, 2, dv, dk, device="cuda") * 0.5 if with_state else None
    _say(io, dk, dv, with_state)
    _run_and_check(w, inp, dout, S0, dF if with_state else None)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_bwd_unbounded_gate(io):
    w = KI.Workload("bwl", 1, 2, 64, 64, 64, 16, io, 1.0, False, 111)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout, dF = (t.cuda() for t in KI.make_grads(w))
    _run_and_check(w, inp, dout, None, dF, gate="logsigmoid")


def test_bwd_batch_and_long_sequence():
    w = KI.Workload("bwb", 2, 2, 2048, 128, 128, 64, "bf16", 4.0, False, 112)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout, dF = (t.cuda() for t in KI.make_grads(w))
    S0 = torch.randn(2, 2, 128, 128, device="cuda") * 0.5
    _run_and_check(w, inp, dout, S0, dF)


def test_bwd_64k_workload_two_heads():
    """The 64k workload at full size (every head computed); heads 0 and 31 checked over all
    65,536 tokens against the oracle's adjoint."""
    w = KI.BY_NAME["64k"]
    _say("64k backward: generating on GPU")
    inp = KI.make_inputs(w, device="cuda")
    dout, dF = KI.make_grads(w, device="cuda")
    _run_and_check(w, inp, dout, None, dF, heads=(0, 31))


def test_autograd_function_matches_the_backward():
    """KdaChunkFunction under torch autograd: loss = sum(dout * out) + sum(dfinal * final_state);
    the gradients autograd hands back are kda_chunk_bwd's, and match the oracle's adjoint."""
    w = KI.Workload("ag", 1, 2, 128, 64, 64, 32, "fp32", 2.0, False, 121)
    inp = {n: t.cuda().requires_grad_(True) for n, t in KI.make_inputs(w).items()}
    dout, dF = (t.cuda() for t in KI.make_grads(w))
    out, fs = kda.KdaChunkFunction.apply(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], -5.0, 32)
    ((out * dout).sum() + (fs * dF).sum()).backward()
    torch.cuda.synchronize()
    x = {n: t.detach().double().cpu().numpy() for n, t in inp.items()}
    ref = native.backward(x["q"], x["k"], x["v"], x["a"], x["beta"], dout.double().cpu().numpy(), -5.0,
                          dfinal=dF.double().cpu().numpy())
    for n, rkey in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("a", "da"), ("beta", "dbeta")):
        _grad_check(inp[n].grad.double().cpu().numpy(), ref[rkey], "fp32", "autograd d" + n)


@pytest.mark.parametrize("io", ["fp32", "bf16"])
def test_bwd_single_chunk_odd_batch_and_heads(io):
    """One 16-token chunk per sequence, B=2 and H=3, dk=128 with dv=64, initial state and final-state
    gradient: the reverse pass runs a single step."""
    w = KI.Workload("bw1", 2, 3, 16, 128, 64, 16, io, 3.0, False, 131)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout, dF = (t.cuda() for t in KI.make_grads(w))
    S0 = torch.randn(2, 3, 64, 128, device="cuda") * 0.5
    _run_and_check(w, inp, dout, S0, dF)


@pytest.mark.parametrize("T", [32, 48, 144])
def test_bwd_short_sequences_and_a_partial_head_group(T):
    """2, 3 and 9 16-token chunks (fewer than the reverse pass's ring holds and than its L2 look-ahead,
    then just past it) over 9 heads (one group of eight heads on an XCD and one partial group), bf16,
    d=128, with an initial state and a final-state gradient: every head against the oracle."""
    w = KI.Workload("bwt%d" % T, 1, 9, T, 128, 128, 16, "bf16", 2.0, False, 140 + T)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout, dF = (t.cuda() for t in KI.make_grads(w))
    S0 = torch.randn(1, 9, 128, 128, device="cuda") * 0.5
    _say("backward short sequence", T)
    _run_and_check(w, inp, dout, S0, dF)


def test_bwd_empty_sequence():
    """No tokens: the only gradient is the initial state's, and it is the final state's."""
    w = KI.Workload("bw0", 1, 2, 0, 64, 64, 16, "bf16", 1.0, False, 132)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    dF = torch.randn(1, 2, 64, 64, device="cuda")
    g = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], dout, dfinal_state=dF)
    torch.cuda.synchronize()
    assert g["dq"].numel() == 0 and g["dbeta"].numel() == 0
    assert torch.equal(g["dinitial_state"], dF)
    g0 = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], dout)
    torch.cuda.synchronize()
    assert not torch.any(g0["dinitial_state"])


@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_bwd_power_of_two_scaling_of_v_is_exact(io):
    # out is linear in v; with dout fixed (and no final-state term) the gradients of q, k, a and
    # beta scale with v and those of v and of the initial state do not depend on it.  Every
    # operand scale inside the backward is a power of two taken from its own block, so scaling v
    # by 2^e changes no rounding: the first group scales by exactly 2^e, the second is unchanged.
    w = KI.Workload("bws", 1, 3, 128, 128, 128, 16, io, 2.0, False, 131)
    _say("backward power-of-two scaling", io)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    dout, _ = (t.cuda() for t in KI.make_grads(w))
    g0 = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], dout)
    for e in (-20, 20):
        x = dict(inp)
        x["v"] = inp["v"] * 2.0 ** e
        g1 = kda.chunk_bwd(x["q"], x["k"], x["v"], x["a"], x["beta"], dout)
        torch.cuda.synchronize()
        for key in ("dq", "dk", "da", "dbeta"):
            assert torch.equal(g1[key], g0[key] * 2.0 ** e), (key, e)
        for key in ("dv", "dinitial_state"):
            assert torch.equal(g1[key], g0[key]), (key, e)
