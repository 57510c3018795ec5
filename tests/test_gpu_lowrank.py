"""Parity of the forward with the gate pre-activation formed in the chunk kernel from a
rank-R factor (kda_chunk_fwd_lowrank, through the C ABI) with the float64 oracle
(oracle.reference.lowrank_preactivation, then the token recurrence), same bar as the
chunked forward: bf16 I/O max|d| <= 2e-2 RMS + u_bf16 |ref| element-wise, fp32 I/O
<= 1e-4 absolute, the final state against the RMS of the oracle's state.

Cases: every chunk size and head-dimension pair with ranks 16 (a half K-block), 32,
64 and 128, both I/O types; an initial state; the unbounded gate of the ablation with
its counters; batches sharing nothing across b; the 64k workload shape at rank 32 at
full size with sampled heads checked in full.
"""
import numpy as np
import pytest
import torch

import chunked_gated_linear_bounded_amd as kda
import kda_inputs as KI
from oracle import native, reference
from parity_util import _say, _tol_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.lib()


def _case(io, T, seed, rank, dk=128, dv=128, chunk=64, B=1, H=2, a_sigma=4.0):
    w = KI.Workload("lr%d" % seed, B, H, T, dk, dv, chunk, io, a_sigma, False, seed)
    inp = {n: t.cuda() for n, t in KI.make_inputs(w).items()}
    lr = {n: t.cuda() for n, t in KI.make_lowrank_factors(w, rank).items()}
    return w, inp, lr


def _run(inp, lr, chunk, **kw):
    return kda.chunk_fwd_lowrank(inp["q"], inp["k"], inp["v"], lr["h"], lr["z"], lr["A_log"], inp["beta"],
                                 chunk=chunk, return_final_state=True, **kw)


def _oracle(inp, lr, gate="bounded", S0=None, heads=None):
    a = reference.lowrank_preactivation(lr["h"].double().cpu().numpy(), lr["z"].double().cpu().numpy(),
                                        lr["A_log"].double().cpu().numpy())
    x = {n: t.double().cpu().numpy() for n, t in inp.items()}
    if heads is not None:
        a = a[:, heads]
        x = {n: t[:, heads] for n, t in x.items()}
    return native.recurrent(x["q"], x["k"], x["v"], a, x["beta"], -5.0, gate=gate, S0=S0)


@pytest.mark.parametrize("io,chunk,dk,dv,rank", [
    ("fp32", 16, 64, 64, 16), ("fp32", 32, 128, 64, 64), ("fp32", 64, 64, 128, 32), ("fp32", 64, 128, 128, 128),
    ("bf16", 16, 128, 128, 32), ("bf16", 32, 64, 128, 16), ("bf16", 64, 128, 128, 128),
    ("bf16", 64, 128, 64, 64), ("bf16", 64, 64, 64, 32), ("bf16", 64, 128, 128, 16),
])
def test_lowrank_parity(io, chunk, dk, dv, rank):
    w, inp, lr = _case(io, 5 * chunk, 81 + rank, rank, dk=dk, dv=dv, chunk=chunk)
    out, fs = _run(inp, lr, chunk)
    torch.cuda.synchronize()
    ro, rf = _oracle(inp, lr)
    _say(io, chunk, dk, dv, rank)
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(fs.double().cpu().numpy(), rf, io, "final_state")


def test_lowrank_batches_and_initial_state():
    w, inp, lr = _case("bf16", 384, 91, 32, B=2, H=3)
    S0 = torch.randn(2, 3, 128, 128, device="cuda") * 0.5
    out, fs = _run(inp, lr, 64, initial_state=S0)
    torch.cuda.synchronize()
    ro, rf = _oracle(inp, lr, S0=S0.double().cpu().numpy())
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")


def test_lowrank_unbounded_gate_counts():
    """The ablation gate through the low-rank path: the fp32 path stays finite and matches the
    oracle; the counters are zeroed-in-place integers and only ever added to."""
    w, inp, lr = _case("fp32", 256, 92, 32, dk=64, dv=64, chunk=16, a_sigma=1.0)
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, fs = _run(inp, lr, 16, gate="logsigmoid", counts=counts)
    torch.cuda.synchronize()
    ro, rf = _oracle(inp, lr, gate="logsigmoid")
    _tol_check(out.double().cpu().numpy(), ro, "fp32")
    assert counts.tolist() == [0, 0]


def test_lowrank_64k_workload_rank32():
    """The 64k workload's shape (H=32, T=65536, d=128, bf16) with the gate from a rank-32 factor,
    launched as the benchmark launches it: heads 0 and 31 checked in full (outputs and final
    state), no non-finite operand or output anywhere."""
    w = KI.BY_NAME["64k"]
    _say("64k lowrank: generating on GPU")
    inp = KI.make_inputs(w, device="cuda")
    lr = KI.make_lowrank_factors(w, 32, device="cuda")
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, fs = _run(inp, lr, 64, counts=counts)
    torch.cuda.synchronize()
    assert counts.tolist() == [0, 0]
    for hd in (0, 31):
        _say(" head", hd)
        sub = {n: t[:, hd:hd + 1] for n, t in inp.items()}
        lsub = {"h": lr["h"], "z": lr["z"][hd:hd + 1], "A_log": lr["A_log"][hd:hd + 1]}
        ro, rf = _oracle(sub, lsub)
        _tol_check(out[:, hd:hd + 1].double().cpu().numpy(), ro, "bf16")
        _tol_check(fs[:, hd:hd + 1].double().cpu().numpy(), rf, "bf16", "final_state")
