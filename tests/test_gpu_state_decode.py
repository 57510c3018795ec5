"""Parity of the initial-state path and of the single-token decode step (through
the C ABI) with the float64 oracle, same bar as the chunked forward: bf16 I/O
max|d| <= 2e-2 RMS + u_bf16 |ref| element-wise, fp32 I/O <= 1e-4 absolute, the
final state against the RMS of the oracle's state.

Cases: a chunked forward from a given state; one sequence processed in two pieces,
the second continuing from the first's final state (also in place); decode steps
from a given state; a chunked prefill continued by decode steps; the unbounded gate
in decode; an empty sequence returning the initial state.
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


def _case(io, T, seed, dk=128, dv=128, chunk=64, a_sigma=4.0, B=1, H=2):
    w = KI.Workload("s%d" % seed, B, H, T, dk, dv, chunk, io, a_sigma, False, seed)
    return w, {n: t.cuda() for n, t in KI.make_inputs(w).items()}


def _state(w, seed, scale=0.5):
    """A seeded initial state [B,H,dv,dk] float32 (stands in for a previous piece's state)."""
    rng = np.random.default_rng(1000 + seed)
    return torch.from_numpy((rng.standard_normal((w.B, w.H, w.dv, w.dk)) * scale).astype(np.float32)).cuda()


def _seg(inp, t0, t1):
    return {n: (t[:, :, t0:t1].contiguous()) for n, t in inp.items()}


def _f64(inp):
    return KI.to_f64({n: t.cpu() for n, t in inp.items()})


@pytest.mark.parametrize("io,chunk", [("fp32", 16), ("fp32", 64), ("bf16", 16), ("bf16", 64)])
def test_chunked_forward_from_initial_state(io, chunk):
    w, inp = _case(io, 5 * chunk, 51, chunk=chunk)
    S0 = _state(w, 51)
    out, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], chunk=chunk,
                            return_final_state=True, initial_state=S0)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], -5.0,
                              S0=S0.double().cpu().numpy())
    _say(io, chunk)
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(fs.double().cpu().numpy(), rf, io, "final_state")


@pytest.mark.parametrize("in_place", [False, True])
def test_sequence_in_two_pieces(in_place):
    w, inp = _case("bf16", 1024, 52)
    p1 = _seg(inp, 0, 384)
    p2 = _seg(inp, 384, 1024)
    o1, f1 = kda.chunk_fwd(p1["q"], p1["k"], p1["v"], p1["a"], p1["beta"], return_final_state=True)
    f2 = f1 if in_place else None
    o2, f2 = kda.chunk_fwd(p2["q"], p2["k"], p2["v"], p2["a"], p2["beta"], return_final_state=True,
                           final_state=f2, initial_state=f1)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], -5.0)
    _tol_check(torch.cat([o1, o2], dim=2).double().cpu().numpy(), ro, "bf16")
    _tol_check(f2.double().cpu().numpy(), rf, "bf16", "final_state")


def _decode(inp, S, t0, t1, gate="bounded"):
    outs = []
    for t in range(t0, t1):
        tok = {n: x[:, :, t].contiguous() for n, x in inp.items()}
        outs.append(kda.decode_step(tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"], S, gate=gate))
    return torch.stack(outs, dim=2)


@pytest.mark.parametrize("io,dk,dv", [("fp32", 64, 64), ("fp32", 128, 64), ("bf16", 64, 128),
                                      ("bf16", 128, 128)])
def test_decode_steps_from_initial_state(io, dk, dv):
    w, inp = _case(io, 48, 53, dk=dk, dv=dv, chunk=16, B=2, H=3)
    S0 = _state(w, 53)
    S = S0.clone()
    out = _decode(inp, S, 0, 48)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], -5.0,
                              S0=S0.double().cpu().numpy())
    _say(io, dk, dv)
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(S.double().cpu().numpy(), rf, io, "state")


def test_prefill_then_decode():
    w, inp = _case("bf16", 320, 54)
    p = _seg(inp, 0, 256)
    o1, S = kda.chunk_fwd(p["q"], p["k"], p["v"], p["a"], p["beta"], return_final_state=True)
    o2 = _decode(inp, S, 256, 320)
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], -5.0)
    _tol_check(torch.cat([o1, o2], dim=2).double().cpu().numpy(), ro, "bf16")
    _tol_check(S.double().cpu().numpy(), rf, "bf16", "state")


def test_decode_unbounded_gate():
    w, inp = _case("fp32", 32, 55, dk=64, dv=64, chunk=16, a_sigma=2.0)
    S0 = _state(w, 55)
    S = S0.clone()
    out = _decode(inp, S, 0, 32, gate="logsigmoid")
    torch.cuda.synchronize()
    i64 = _f64(inp)
    ro, rf = native.recurrent(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], -5.0, gate="logsigmoid",
                              S0=S0.double().cpu().numpy())
    _tol_check(out.double().cpu().numpy(), ro, "fp32")
    _tol_check(S.double().cpu().numpy(), rf, "fp32", "state")


def test_empty_sequence_keeps_the_initial_state():
    w, inp = _case("bf16", 0, 56)
    S0 = _state(w, 56)
    out, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], return_final_state=True,
                            initial_state=S0)
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert torch.equal(fs, S0)
