"""Seeded input generators: reproducible, with the workloads' distributions."""
import numpy as np
import torch

import kda_inputs as KI


def test_workload_table():
    names = [w.name for w in KI.WORKLOADS]
    assert names == ["tiny", "8k", "64k", "256k", "1m"]
    assert [w.seed for w in KI.WORKLOADS] == [0, 1, 2, 3, 4]
    w = KI.BY_NAME["64k"]
    assert (w.B, w.H, w.T, w.dk, w.dv, w.chunk, w.io) == (1, 32, 65536, 128, 128, 64, "bf16")


def test_reproducible_and_normalised():
    w = KI.BY_NAME["tiny"]
    x1 = KI.make_inputs(w)
    x2 = KI.make_inputs(w)
    for n in x1:
        assert torch.equal(x1[n], x2[n])
        assert x1[n].dtype == torch.float32
    nq = torch.linalg.vector_norm(x1["q"].double(), dim=-1)
    assert torch.allclose(nq, torch.ones_like(nq), atol=1e-6)
    b = x1["beta"]
    assert float(b.min()) > 0 and float(b.max()) < 1
    x3 = KI.make_inputs(w.with_(seed=9))
    assert not torch.equal(x1["q"], x3["q"])


def test_bf16_and_mixture():
    w = KI.BY_NAME["1m"].with_(T=4096, H=2)
    x = KI.make_inputs(w)
    assert x["a"].dtype == torch.bfloat16
    a = x["a"].float()
    frac = float((a.abs() == 12.0).float().mean())
    assert 0.09 < frac < 0.11
    assert abs(float((a == 12.0).float().mean()) - float((a == -12.0).float().mean())) < 0.01
    nk = torch.linalg.vector_norm(x["k"].double(), dim=-1)
    assert float((nk - 1).abs().max()) < 2 ** -7


def test_gate_spread_of_64k():
    # a ~ N(0, 4^2): about 16.5% of the bounded gates sit below -4.9
    w = KI.BY_NAME["64k"].with_(T=2048, H=2)
    a = KI.make_inputs(w)["a"].double().numpy()
    g = -5.0 / (1.0 + np.exp(-a))
    assert 0.14 < float((g < -4.9).mean()) < 0.19
