"""Seeded synthetic inputs for the KDA chunked forward (shared by tests, bench, smoke).

This module holds no arithmetic of the method: it only draws random tensors of
the shapes and distributions of the workloads below and rounds them to the I/O
dtype.  Both the oracle side and the GPU side consume what it returns.

Workloads (the pages' staged context lengths 8K -> 64K -> 256K -> 1M, "Trillion-
Scale MoE Multimodal Models: Practical Techniques ...", sec. 2.3; no dataset is
involved, seeded synthetic tensors stand in for the training sequences):

  tiny   B=1  H=2  T=256      dk=dv=64  chunk=16 fp32  a ~ N(0,1)
  8k     B=4  H=16 T=8192     dk=dv=128 chunk=64 bf16  a ~ N(0,2^2)
  64k    B=1  H=32 T=65536    dk=dv=128 chunk=64 bf16  a ~ N(0,4^2)   (throughput workload)
  256k   B=1  H=16 T=262144   dk=dv=128 chunk=64 bf16  a ~ N(0,4^2)   (+ final state)
  1m     B=1  H=8  T=1048576  dk=dv=128 chunk=64 bf16  a ~ 0.9 N(0,1) + 0.1 (+-12)
                                                         (+ unbounded-gate ablation)

For all: q, k ~ N(0,1) then L2-normalised over dk per (head, token) in float64;
v ~ N(0,1); beta = sigmoid(N(0,1)); g_min = -5.  Workload i uses seed i.

Streams: on the CPU every (tensor, b, h) slab has its own PCG64 stream from
numpy.random.SeedSequence([seed, tensor_id, b, h]) with tensor ids
q=0, k=1, v=2, a=3, beta=4, mixture-mask=5, mixture-sign=6.  On a GPU device the
same per-slab seeds drive torch's device generator (faster for the large
workloads); the two devices give different but each reproducible values, and
every comparison hands the oracle exactly the tensors the GPU consumed.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "a": 3, "beta": 4, "mix_mask": 5, "mix_sign": 6,
              "lr_h": 8, "lr_z": 9, "lr_A": 10, "dout": 11, "dfinal": 12}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    io: str            # "fp32" or "bf16"
    a_sigma: float     # std of the gate pre-activation (when not a mixture)
    a_mixture: bool    # 0.9 N(0,1) + 0.1 (+-12)
    seed: int
    g_min: float = -5.0
    final_state: bool = False
    ablation: bool = False

    @property
    def torch_dtype(self):
        return torch.float32 if self.io == "fp32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = [
    Workload("tiny", 1, 2, 256, 64, 64, 16, "fp32", 1.0, False, 0),
    Workload("8k", 4, 16, 8192, 128, 128, 64, "bf16", 2.0, False, 1),
    Workload("64k", 1, 32, 65536, 128, 128, 64, "bf16", 4.0, False, 2),
    Workload("256k", 1, 16, 262144, 128, 128, 64, "bf16", 4.0, False, 3, final_state=True),
    Workload("1m", 1, 8, 1048576, 128, 128, 64, "bf16", 1.0, True, 4, ablation=True),
]
BY_NAME = {w.name: w for w in WORKLOADS}


def _slab_seed(seed, name, b, h):
    return np.random.SeedSequence([seed, TENSOR_IDS[name], b, h])


def _draw_cpu(seed, name, b, h, n):
    return np.random.Generator(np.random.PCG64(_slab_seed(seed, name, b, h))).standard_normal(n)


def _draw_dev(seed, name, b, h, n, device):
    s = int(_slab_seed(seed, name, b, h).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
    gen = torch.Generator(device=device)
    gen.manual_seed(s)
    return torch.randn(n, generator=gen, device=device, dtype=torch.float32)


def _uniform_dev(seed, name, b, h, n, device):
    s = int(_slab_seed(seed, name, b, h).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))
    gen = torch.Generator(device=device)
    gen.manual_seed(s)
    return torch.rand(n, generator=gen, device=device, dtype=torch.float32)


def make_inputs(w: Workload, device="cpu"):
    """Returns dict q, k, v, a, beta of torch tensors in the workload's I/O dtype,
    shapes q,k,a [B,H,T,dk], v [B,H,T,dv], beta [B,H,T], on `device`."""
    device = torch.device(device)
    dt = w.torch_dtype
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    out = {n: torch.empty(shape, dtype=dt, device=device) for n, shape in
           (("q", (B, H, T, dk)), ("k", (B, H, T, dk)), ("v", (B, H, T, dv)),
            ("a", (B, H, T, dk)), ("beta", (B, H, T)))}
    for b in range(B):
        for h in range(H):
            if device.type == "cpu":
                for n, d in (("q", dk), ("k", dk)):
                    x = _draw_cpu(w.seed, n, b, h, T * d).reshape(T, d)
                    x /= np.linalg.norm(x, axis=1, keepdims=True)
                    out[n][b, h] = torch.from_numpy(x).to(dt)
                out["v"][b, h] = torch.from_numpy(_draw_cpu(w.seed, "v", b, h, T * dv).reshape(T, dv)).to(dt)
                a = _draw_cpu(w.seed, "a", b, h, T * dk).reshape(T, dk) * w.a_sigma
                if w.a_mixture:
                    gm = np.random.Generator(np.random.PCG64(_slab_seed(w.seed, "mix_mask", b, h)))
                    gs = np.random.Generator(np.random.PCG64(_slab_seed(w.seed, "mix_sign", b, h)))
                    outlier = gm.random((T, dk)) < 0.1
                    sign = np.where(gs.random((T, dk)) < 0.5, -1.0, 1.0)
                    a = np.where(outlier, 12.0 * sign, a)
                out["a"][b, h] = torch.from_numpy(a).to(dt)
                z = _draw_cpu(w.seed, "beta", b, h, T)
                out["beta"][b, h] = torch.from_numpy(1.0 / (1.0 + np.exp(-z))).to(dt)
            else:
                for n, d in (("q", dk), ("k", dk)):
                    x = _draw_dev(w.seed, n, b, h, T * d, device).view(T, d)
                    x = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
                    out[n][b, h] = x.to(dt)
                out["v"][b, h] = _draw_dev(w.seed, "v", b, h, T * dv, device).view(T, dv).to(dt)
                a = _draw_dev(w.seed, "a", b, h, T * dk, device).view(T, dk) * w.a_sigma
                if w.a_mixture:
                    outlier = _uniform_dev(w.seed, "mix_mask", b, h, T * dk, device).view(T, dk) < 0.1
                    sign = torch.where(_uniform_dev(w.seed, "mix_sign", b, h, T * dk, device).view(T, dk) < 0.5,
                                       -1.0, 1.0)
                    a = torch.where(outlier, 12.0 * sign, a)
                    del outlier, sign
                out["a"][b, h] = a.to(dt)
                z = _draw_dev(w.seed, "beta", b, h, T, device)
                out["beta"][b, h] = torch.sigmoid(z).to(dt)
    return out


# Packed documents (short documents laid end to end in one long sequence, "Breaking
# Through Trillion-Parameter Multimodal MoE ...", sec. 3, 256K-1M phase): document
# lengths drawn log-uniformly in [lo, hi] from PCG64(SeedSequence([seed, 7])) until
# they fill T, the last one cut to fit.  The token tensors are those of a B=1
# workload of the same seed, with the batch axis dropped: [H, T, d].
PACKED = Workload("packed64k", 1, 32, 65536, 128, 128, 64, "bf16", 4.0, False, 5)
PACKED_LEN = (32, 4096)


def packed_lengths(T, seed, lo=PACKED_LEN[0], hi=PACKED_LEN[1]):
    """Document lengths (ints >= 1 unless T == 0) that sum to T."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    lens, total = [], 0
    while total < T:
        n = int(np.exp(rng.uniform(np.log(lo), np.log(hi + 1))))
        n = max(1, min(n, T - total))
        lens.append(n)
        total += n
    return lens


def cu_seqlens(lengths):
    """int32 boundaries [0, l0, l0 + l1, ...] of documents of the given lengths."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def make_packed_inputs(w: Workload, device="cpu"):
    """Token tensors of a packed stream: q, k, a [H,T,dk]; v [H,T,dv]; beta [H,T]."""
    assert w.B == 1
    return {n: t[0] for n, t in make_inputs(w, device).items()}


# Gate pre-activation from a rank-R factor: h [B,T,R] ~ N(0,1) (one slab per batch, shared by
# the heads), z [H,dk,R] ~ N(0,1)/sqrt(R) (one slab per head), both rounded to the I/O dtype,
# and A_log [H,dk] = ln(a_sigma) + 0.25 N(0,1) in float32, so that the pre-activation
# e^A (h z) has about the workload's a_sigma spread.  Streams as above (ids 8, 9, 10).
def make_lowrank_factors(w: Workload, rank: int, device="cpu"):
    device = torch.device(device)
    dt = w.torch_dtype
    h = torch.empty((w.B, w.T, rank), dtype=dt, device=device)
    z = torch.empty((w.H, w.dk, rank), dtype=dt, device=device)
    A = torch.empty((w.H, w.dk), dtype=torch.float32, device=device)
    draw = (lambda name, b, hh, n: torch.from_numpy(_draw_cpu(w.seed, name, b, hh, n)).to(device)) \
        if device.type == "cpu" else (lambda name, b, hh, n: _draw_dev(w.seed, name, b, hh, n, device))
    for b in range(w.B):
        h[b] = draw("lr_h", b, 0, w.T * rank).view(w.T, rank).to(dt)
    for hh in range(w.H):
        z[hh] = (draw("lr_z", 0, hh, w.dk * rank).view(w.dk, rank) / np.sqrt(rank)).to(dt)
        A[hh] = (np.log(w.a_sigma) + 0.25 * draw("lr_A", 0, hh, w.dk)).to(torch.float32)
    return {"h": h, "z": z, "A_log": A}


# Incoming gradients for the backward: dout [B,H,T,dv] ~ N(0,1) in the I/O dtype and dfinal
# [B,H,dv,dk] ~ 0.1 N(0,1) in float32, per (b, h) slab (ids 11, 12).
def make_grads(w: Workload, device="cpu"):
    device = torch.device(device)
    dout = torch.empty((w.B, w.H, w.T, w.dv), dtype=w.torch_dtype, device=device)
    dfin = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=device)
    for b in range(w.B):
        for h in range(w.H):
            if device.type == "cpu":
                dout[b, h] = torch.from_numpy(_draw_cpu(w.seed, "dout", b, h, w.T * w.dv).reshape(w.T, w.dv)).to(
                    w.torch_dtype)
                dfin[b, h] = torch.from_numpy(0.1 * _draw_cpu(w.seed, "dfinal", b, h, w.dv * w.dk).reshape(
                    w.dv, w.dk)).to(torch.float32)
            else:
                dout[b, h] = _draw_dev(w.seed, "dout", b, h, w.T * w.dv, device).view(w.T, w.dv).to(w.torch_dtype)
                dfin[b, h] = 0.1 * _draw_dev(w.seed, "dfinal", b, h, w.dv * w.dk, device).view(w.dv, w.dk)
    return dout, dfin


def head_slice(inputs, b, h, t_end=None, t_start=None):
    """float64 NumPy copies of one (b, h) head's inputs (tokens t_start .. t_end - 1, default
    all), with leading singleton B and H axes, for the oracle."""
    sl = slice(t_start, t_end)
    res = {}
    for n in ("q", "k", "v", "a"):
        res[n] = inputs[n][b:b + 1, h:h + 1, sl].detach().to("cpu", torch.float64).numpy()
    res["beta"] = inputs["beta"][b:b + 1, h:h + 1, sl].detach().to("cpu", torch.float64).numpy()
    return res


def to_f64(inputs):
    """float64 NumPy copies of all inputs."""
    return {n: t.detach().to("cpu", torch.float64).numpy() for n, t in inputs.items()}
