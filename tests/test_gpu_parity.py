"""Parity of the HIP path (through the C ABI) with the float64 oracle.

Bar, element by element (tests/parity_util.py):
  bf16 I/O  |out - oracle| <= 2e-2 * RMS(oracle out) + 2^-8 * |oracle out|
            -- the stated 2e-2 RMS bound on the computation, plus the one rounding of the exact
            result to bf16 that every bf16 output carries (half an ulp, at most 2^-8 relative).
            The literal max|d|/RMS is printed beside it: rounding alone exceeds 2e-2 RMS wherever
            |out| > 5.12 RMS, which heavy-tailed outputs reach.
  fp32 I/O  |out - oracle| <= 1e-4 absolute.
The final state (float32) follows the bf16 rule against RMS(oracle state) with bf16 inputs.
Small problems here are compared in full; the four large workloads are compared head by head over
every output in tests/test_gpu_workloads.py.
"""

import numpy as np
import pytest
import torch

import chunked_gated_linear_bounded_amd as kda
import kda_inputs as KI
from oracle import native, reference

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.lib()


from parity_util import _say, _tol_check  # noqa: E402


def _gpu_run(inp, chunk, g_min=-5.0, gate="bounded", counts=None):
    return kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], g_min=g_min, chunk=chunk,
                         return_final_state=True, gate=gate, counts=counts)


def _oracle(inp64, g_min=-5.0, gate="bounded"):
    return native.recurrent(inp64["q"], inp64["k"], inp64["v"], inp64["a"], inp64["beta"], g_min, gate=gate)


def _to_dev(inp):
    return {n: t.cuda() for n, t in inp.items()}


# ---------------------------------------------------------------- gate kernel
@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("chunk,dk", [(16, 64), (32, 128), (64, 128), (64, 64)])
@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
def test_gate_cumsum(io, chunk, dk, gate):
    w = KI.Workload("g", 2, 3, 4 * chunk, dk, dk, chunk, io, 4.0, True, 17)
    _say("gate_cumsum", io, chunk, dk, gate)
    inp = _to_dev(KI.make_inputs(w))
    G = kda.gate_cumsum(inp["a"], -5.0, chunk, gate=gate)
    torch.cuda.synchronize()
    a64 = inp["a"].double().cpu().numpy()
    g = reference.gate(a64, -5.0, gate)
    want = np.concatenate([np.cumsum(g[:, :, n0:n0 + chunk], axis=2) for n0 in range(0, w.T, chunk)], axis=2)
    got = G.double().cpu().numpy()
    err = np.abs(got - want)
    assert np.all(err <= 1e-4 + 2e-6 * np.abs(want)), float(err.max())


# ---------------------------------------------------------------- all shapes, small sizes, full compare
SHAPES = [(dk, dv, c) for dk in (64, 128) for dv in (64, 128) for c in (16, 32, 64)]


@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv,chunk", SHAPES)
def test_small_parity_all_shapes(io, dk, dv, chunk):
    # several chunks, a head count that leaves the last group of 8 heads ragged
    w = KI.Workload("s", 1, 3, 5 * chunk, dk, dv, chunk, io, 2.0, False, 100 + dk + dv + chunk)
    _say("small", io, dk, dv, chunk)
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, chunk)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(fs.double().cpu().numpy(), rf, io, "final_state")


def test_tiny_workload_full():
    w = KI.BY_NAME["tiny"]
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, w.chunk)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, "fp32")
    _tol_check(fs.double().cpu().numpy(), rf, "fp32", "final_state")


def test_multi_batch_bf16():
    w = KI.Workload("mb", 3, 5, 384, 128, 128, 64, "bf16", 4.0, False, 55)
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, 64)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")


@pytest.mark.parametrize("nchunks", [1, 2, 3, 4, 5, 9])
def test_sequences_around_the_prefetch_distance(nchunks):
    # bf16, d = 128, chunk 64: the state stage touches each record four chunks ahead of its LDS
    # ring; sequences shorter than, equal to and longer than that distance, 12 heads (a ragged
    # group of 8 heads on the last XCD)
    w = KI.Workload("pf", 1, 12, 64 * nchunks, 128, 128, 64, "bf16", 4.0, False, 300 + nchunks)
    _say("prefetch distance", nchunks)
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, 64)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")


# ---------------------------------------------------------------- invariants
def test_beta_zero_exact_zero():
    w = KI.Workload("z", 1, 2, 256, 128, 128, 64, "bf16", 4.0, False, 3)
    inp = _to_dev(KI.make_inputs(w))
    inp["beta"].zero_()
    out, fs = _gpu_run(inp, 64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0 and torch.count_nonzero(fs).item() == 0


def test_delta_retrieval_fp32():
    w = KI.Workload("d", 1, 2, 256, 64, 64, 16, "fp32", 2.0, False, 4)
    inp = _to_dev(KI.make_inputs(w))
    inp["q"] = inp["k"].clone()
    inp["beta"].fill_(1.0)
    out, _ = _gpu_run(inp, 16)
    torch.cuda.synchronize()
    assert float((out - inp["v"]).abs().max()) <= 1e-4


def test_deterministic_and_causal():
    w = KI.Workload("c", 1, 4, 512, 128, 128, 64, "bf16", 4.0, False, 8)
    inp = _to_dev(KI.make_inputs(w))
    o1, f1 = _gpu_run(inp, 64)
    o2, f2 = _gpu_run(inp, 64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    t = 5 * 64 + 17  # inside chunk 5
    inp["k"][:, :, t] = -inp["k"][:, :, t]
    inp["v"][:, :, t] = 3.0
    o3, _ = _gpu_run(inp, 64)
    torch.cuda.synchronize()
    assert torch.equal(o3[:, :, :t], o1[:, :, :t])
    assert not torch.equal(o3[:, :, t:], o1[:, :, t:])


def test_chunk_sizes_agree():
    w = KI.Workload("cs", 1, 2, 512, 128, 128, 64, "bf16", 4.0, False, 9)
    inp = _to_dev(KI.make_inputs(w))
    ro, _ = _oracle(KI.to_f64(inp))
    for c in (16, 32, 64):
        o, _ = _gpu_run(inp, c)
        torch.cuda.synchronize()
        _tol_check(o.double().cpu().numpy(), ro, "bf16", "out chunk %d" % c)


def test_linear_in_v():
    w = KI.Workload("lv", 1, 2, 256, 64, 64, 32, "fp32", 2.0, False, 10)
    x = _to_dev(KI.make_inputs(w))
    y = dict(x)
    y["v"] = torch.randn_like(x["v"])
    z = dict(x)
    z["v"] = 2.0 * x["v"] - 3.0 * y["v"]
    ox, _ = _gpu_run(x, 32)
    oy, _ = _gpu_run(y, 32)
    oz, _ = _gpu_run(z, 32)
    torch.cuda.synchronize()
    assert float((oz - (2.0 * ox - 3.0 * oy)).abs().max()) <= 1e-4


@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("chunk", [16, 64])
def test_power_of_two_scaling_of_v_is_exact(io, chunk):
    # Every 16-bit operand that follows the scale of v is scaled by a power of two taken from its
    # own block, so scaling v by 2^e changes no rounding: out and the final state scale by exactly
    # 2^e, far beyond the fp16 range in both directions.
    w = KI.Workload("p2", 1, 3, 4 * chunk, 128, 128, chunk, io, 4.0, False, 77 + chunk)
    _say("power-of-two scaling", io, chunk)
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, chunk)
    for e in (-20, 20):
        x = dict(inp)
        x["v"] = inp["v"] * 2.0 ** e
        o2, f2 = _gpu_run(x, chunk)
        torch.cuda.synchronize()
        assert torch.equal(o2.float(), out.float() * 2.0 ** e), (e, float((o2.float() - out.float() * 2.0 ** e).abs().max()))
        assert torch.equal(f2, fs * 2.0 ** e), e


def test_value_scale_jumping_between_chunks():
    # v's magnitude jumps by up to 2^8 from one chunk to the next, so the state's largest
    # magnitude leaves the window its scale is kept in, upwards and downwards, many times: the
    # state stage then forms the wave-wide maximum and rescales, where at other chunks it only
    # checks the window with lane masks.  Chunk by chunk against the oracle, each chunk held to
    # the bound relative to its own RMS.
    w = KI.Workload("jump", 1, 3, 64 * 12, 128, 128, 64, "bf16", 1.0, False, 913)
    _say("value scale jumping between chunks")
    inp = _to_dev(KI.make_inputs(w))
    e = torch.tensor([0, 8, -8, 4, -4, 8, 8, -8, -8, 0, 6, -6], dtype=torch.float32, device="cuda")
    scale = torch.exp2(e).repeat_interleave(64)  # per token; powers of two are exact in bf16
    inp["v"] = (inp["v"].float() * scale[None, None, :, None]).to(inp["v"].dtype)
    out, fs = _gpu_run(inp, 64)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    got = out.double().cpu().numpy()
    for n in range(12):
        _tol_check(got[:, :, 64 * n:64 * n + 64], ro[:, :, 64 * n:64 * n + 64], "bf16", "chunk %d" % n)
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")


@pytest.mark.parametrize("B,H,T,d,chunk,nseg", [(2, 128, 256, 64, 16, 1), (1, 5, 64 * 40, 128, 64, 40 // 8),
                                               (1, 3, 32 * 85, 128, 32, 10)])
def test_state_stage_segment_layouts(B, H, T, d, chunk, nseg):
    # 256 heads: the segmented stage with one segment (pass 1 alone, one work-group per head);
    # 5 heads x 40 chunks: 5 segments of 8 chunks; 3 heads x 85 chunks: 10 segments of 9, the last
    # one of 4 (segments are never empty) -- every output and final state against the oracle
    w = KI.Workload("seg", B, H, T, d, d, chunk, "bf16", 4.0, False, 600 + H)
    _say("segment layout", B, H, T, d, chunk, nseg)
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, chunk)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, "bf16")
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")


@pytest.mark.parametrize("path", ["segmented", "noalloc", "packed"])
def test_state_that_decays_to_nothing_then_takes_new_values(path):
    # From a random initial state, eight chunks with v = 0 under saturated gates (g = g_min, a decay
    # of e^-320 per channel and chunk) take the state far below the float32 range, then ordinary
    # chunks follow.  The state stage keeps the state as a scaled mantissa and an integer exponent,
    # so its exponent grows by hundreds; the products of the next chunk must stay finite and exact
    # (the oracle's state is exactly zero by then in float64 too).  24 chunks: the segmented stage
    # walks three segments of 8 (the quiet stretch covers a whole segment); the allocation-free and
    # packed forwards use the per-slice stage.
    w = KI.Workload("decay", 1, 2, 64 * 24, 128, 128, 64, "bf16", 2.0, False, 515)
    _say("decayed state then new values", path)
    inp = _to_dev(KI.make_inputs(w))
    quiet = slice(64 * 4, 64 * 12)
    inp["v"][:, :, quiet] = 0
    inp["a"][:, :, quiet] = 12.0
    g = torch.Generator(device="cpu").manual_seed(5151)
    s0 = torch.randn((1, 2, 128, 128), generator=g, dtype=torch.float64).float().cuda()
    if path == "segmented":
        out, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], chunk=64,
                                return_final_state=True, initial_state=s0)
    elif path == "noalloc":
        out = torch.empty_like(inp["v"])
        fs = torch.empty_like(s0)
        kda.chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], out, chunk=64, final_state=fs,
                              initial_state=s0)
    else:
        cu = torch.tensor([0, w.T], dtype=torch.int32, device="cuda")
        o, f = kda.chunk_fwd_varlen(inp["q"][0], inp["k"][0], inp["v"][0], inp["a"][0], inp["beta"][0], cu, chunk=64,
                                    return_final_state=True, initial_state=s0.reshape(1, 2, 128, 128))
        out, fs = o[None], f.reshape(1, 2, 128, 128)
    torch.cuda.synchronize()
    i64 = KI.to_f64(inp)
    ro, rf = native.recurrent(i64["q"], i64["k"], i64["v"], i64["a"], i64["beta"], -5.0, S0=s0.double().cpu().numpy())
    got = out.double().cpu().numpy()
    assert np.all(np.isfinite(got))
    _tol_check(got, ro, "bf16", "whole sequence")
    for n in range(12, 24):  # the chunks after the quiet stretch, each against its own RMS
        _tol_check(got[:, :, 64 * n:64 * n + 64], ro[:, :, 64 * n:64 * n + 64], "bf16", "chunk %d" % n)
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")


@pytest.mark.parametrize("path", ["segmented", "noalloc"])
def test_state_exactly_zero_for_the_first_chunks(path):
    # v = 0 for the first five chunks: from a zero initial state the state stays exactly zero
    # (its range check finds a zero maximum), so the fp16 scale of U comes from the bound on U~
    # alone until values arrive.  Against the oracle, and scaling v by 2^-20 or 2^20 scales every
    # output and the final state exactly.  The allocation-free forward uses the per-slice stage,
    # the plain one at two heads the segmented stage (24 chunks: three segments, each of whose
    # local chains in pass 0 also starts from a zero state, beside the transition chains).
    w = KI.Workload("zlead", 1, 2, 64 * 24, 128, 128, 64, "bf16", 2.0, False, 717)
    _say("state exactly zero for the first chunks", path)
    inp = _to_dev(KI.make_inputs(w))
    inp["v"][:, :, :64 * 5] = 0

    def run(x):
        if path == "segmented":
            return kda.chunk_fwd(x["q"], x["k"], x["v"], x["a"], x["beta"], chunk=64, return_final_state=True)
        out = torch.empty_like(x["v"])
        fs = torch.empty((1, 2, 128, 128), dtype=torch.float32, device="cuda")
        kda.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["a"], x["beta"], out, chunk=64, final_state=fs)
        return out, fs

    out, fs = run(inp)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    got = out.double().cpu().numpy()
    assert np.all(got[:, :, :64 * 5] == 0)
    _tol_check(got, ro, "bf16", "whole sequence")
    for n in range(5, 24):
        _tol_check(got[:, :, 64 * n:64 * n + 64], ro[:, :, 64 * n:64 * n + 64], "bf16", "chunk %d" % n)
    _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")
    for e in (-20, 20):
        x = dict(inp)
        x["v"] = inp["v"] * 2.0 ** e
        o2, f2 = run(x)
        torch.cuda.synchronize()
        assert torch.equal(o2.float(), out.float() * 2.0 ** e), e
        assert torch.equal(f2, fs * 2.0 ** e), e


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("bf16", 16), ("fp32", 64)])
def test_every_gate_saturated_at_the_bound(io, chunk):
    # a = +12 everywhere: every g sits at g_min = -5, the most negative value accepted, so the
    # diagonal sub-tiles' key factors reach e^75 and their row factors e^-75 -- the extreme
    # the bound allows, checked element by element against the oracle
    w = KI.Workload("sat", 1, 3, 4 * 64, 128, 128, chunk, io, 1.0, False, 41)
    _say("saturated gates", io, chunk)
    inp = _to_dev(KI.make_inputs(w))
    inp["a"] = torch.full_like(inp["a"], 12.0)
    counts = torch.zeros(2, dtype=torch.int64, device="cuda")
    out, fs = _gpu_run(inp, chunk, counts=counts)
    torch.cuda.synchronize()
    assert counts.tolist() == [0, 0]
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(fs.double().cpu().numpy(), rf, io, "final_state")


def test_empty_sequence():
    inp = {n: torch.empty((1, 2, 0, 64) if n != "beta" else (1, 2, 0), dtype=torch.bfloat16, device="cuda")
           for n in ("q", "k", "v", "a", "beta")}
    out, fs = _gpu_run(inp, 16)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64) and torch.count_nonzero(fs).item() == 0


@pytest.mark.parametrize("io,chunk", [("bf16", 64), ("bf16", 16), ("fp32", 32)])
def test_unnormalised_queries_and_keys(io, chunk):
    # q and k off the unit sphere: q x 8 and k x 1.3 (beta |k|^2 <= 1.69 < 2 keeps every step of the
    # delta rule a contraction, so the recurrence itself stays bounded).  Every fp16 operand inside
    # the chunk stage is block-scaled, so nothing depends on |q| |k| <= 1.
    w = KI.Workload("unorm", 1, 3, 6 * 64, 128, 128, chunk, io, 4.0, False, 515)
    _say("unnormalised q, k", io, chunk)
    inp = _to_dev(KI.make_inputs(w))
    inp["q"] = (inp["q"].float() * 8.0).to(inp["q"].dtype)
    inp["k"] = (inp["k"].float() * 1.3).to(inp["k"].dtype)
    out, fs = _gpu_run(inp, chunk)
    torch.cuda.synchronize()
    ro, rf = _oracle(KI.to_f64(inp))
    _tol_check(out.double().cpu().numpy(), ro, io)
    _tol_check(fs.double().cpu().numpy(), rf, io, "final_state")


@pytest.mark.parametrize("e", [-12, 12])
def test_power_of_two_scaling_of_q_is_exact(e):
    # q enters M and Q e^G linearly, and both are block-scaled by powers of two: scaling q by 2^e
    # scales out by exactly 2^e and leaves the final state unchanged
    w = KI.Workload("q2", 1, 3, 4 * 64, 128, 128, 64, "bf16", 4.0, False, 616)
    inp = _to_dev(KI.make_inputs(w))
    out, fs = _gpu_run(inp, 64)
    x = dict(inp)
    x["q"] = inp["q"] * 2.0 ** e
    o2, f2 = _gpu_run(x, 64)
    torch.cuda.synchronize()
    assert torch.equal(o2.float(), out.float() * 2.0 ** e)
    assert torch.equal(f2, fs)


def test_side_stream_with_library_allocations():
    # chunk_fwd on a stream other than the current one, with out, final state and workspace
    # allocated by the binding: the current stream allocates and fills tensors of the same sizes at
    # once, which must not receive any of those blocks while the kernels still use them
    w = KI.Workload("side", 1, 8, 16 * 64, 128, 128, 64, "bf16", 4.0, False, 717)
    inp = _to_dev(KI.make_inputs(w))
    ro, rf = _oracle(KI.to_f64(inp))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], chunk=64,
                                  return_final_state=True, stream=side))
        junk = [torch.full((w.B, w.H, w.T, w.dv), 7.0, dtype=torch.bfloat16, device="cuda"),
                torch.full((kda.workspace_bytes(w.B, w.H, w.T, w.dk, w.dv, 64, torch.bfloat16),), 255,
                           dtype=torch.uint8, device="cuda")]
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for out, fs in outs:
        _tol_check(out.double().cpu().numpy(), ro, "bf16")
        _tol_check(fs.double().cpu().numpy(), rf, "bf16", "final_state")
