"""Every output of every large workload against the float64 oracle.

The four bf16 workloads (the pages' context stages 8K, 64K, 256K and 1M, "Trillion-Scale MoE
Multimodal Models: Practical Techniques ...", sec. 2.3) run once each on the GPU through the C ABI,
in the launch configuration the benchmark times.  Then every head is compared element by element
with the oracle over its whole sequence, together with its final state: 64 heads of 8k, 32 of 64k,
16 of 256k and 8 of 1m.  The oracle runs a long head in pieces of 2^17 tokens, each continued from
the previous piece's final state.  That is the same float64 recurrence as one run, since the state
is carried over exactly.

Bar (tests/parity_util.py): bf16 output |d| <= 2e-2 RMS(ref) + 2^-8 |ref| per element.  That is the
stated 2e-2 RMS bound on the computation plus the one rounding of the exact result to bf16.  The
final state (float32) uses the same rule against its own RMS.  Each head prints the literal
max|d|/RMS, the excess over the rounding allowance and RMS(d)/RMS; each workload's summary prints
the worst of every head.

The 1m workload also runs with the unbounded log-sigmoid gate (the ablation of "Breaking Through
Trillion-Parameter Multimodal MoE ...", sec. 2.1).  Its count of non-finite bf16 Gamma-scaled
operands is compared, at full size, with the CPU predictor, which is streamed per head and piece.
The bounded run of the same inputs must count none.
"""
import concurrent.futures as cf

import pytest
import torch

import chunked_gated_linear_bounded_amd as kda
import kda_inputs as KI
from oracle import native, overflow
from parity_util import StreamCheck, _say

pytestmark = pytest.mark.gpu

PIECE = 1 << 17  # tokens per oracle call
NAMES = ("8k", "64k", "256k", "1m")
_CACHE = {}
_STATS = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kda.lib()
    yield
    _CACHE.clear()
    torch.cuda.empty_cache()


def _run(name):
    """Inputs, out and final state of workload `name` on the GPU (one workload cached at a time)."""
    if name not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        w = KI.BY_NAME[name]
        _say("workload", name, "B=%d H=%d T=%d: generating on the GPU" % (w.B, w.H, w.T))
        inp = KI.make_inputs(w, device="cuda")
        counts = torch.zeros(2, dtype=torch.int64, device="cuda")
        out, fs = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], g_min=w.g_min,
                                chunk=w.chunk, return_final_state=True, counts=counts)
        torch.cuda.synchronize()
        _CACHE[name] = (w, inp, out, fs, counts.tolist())
    return _CACHE[name]


ITEMS = []
for _n in NAMES:
    _w = KI.BY_NAME[_n]
    ITEMS += [("head", _n, b, h) for b in range(_w.B) for h in range(_w.H)]
    ITEMS.append(("summary", _n, -1, -1))


@pytest.mark.parametrize("kind,name,b,h", ITEMS,
                         ids=["%s-%s" % (n, "b%dh%d" % (b, h) if k == "head" else "all") for k, n, b, h in ITEMS])
def test_workload_every_output(kind, name, b, h):
    w, inp, out, fs, counts = _run(name)
    if kind == "summary":
        st = _STATS.get(name, {})
        assert len(st) == w.B * w.H, "%d of %d heads compared" % (len(st), w.B * w.H)
        for key in ("out", "final_state"):
            worst = {f: max(s[key][f] for s in st.values()) for f in ("literal", "excess", "rel_rms",
                                                                      "max_ref_over_rms")}
            _say("SUMMARY %s %s heads=%d literal=%.3e excess=%.3e rel_rms=%.3e max_ref_over_rms=%.1f" % (
                name, key, len(st), worst["literal"], worst["excess"], worst["rel_rms"], worst["max_ref_over_rms"]))
        assert counts == [0, 0], "bounded gate: non-finite operands or outputs %s" % counts
        return
    _say("head", name, b, h)
    chk = StreamCheck(w.io, "%s b%d h%d out" % (name, b, h))
    S = None
    for t0 in range(0, w.T, PIECE):
        t1 = min(w.T, t0 + PIECE)
        hs = KI.head_slice(inp, b, h, t1, t0)
        ro, S = native.recurrent(hs["q"], hs["k"], hs["v"], hs["a"], hs["beta"], w.g_min, S0=S)
        chk.add(out[b, h, t0:t1].double().cpu().numpy(), ro[0, 0])
    so = chk.finish()
    chk = StreamCheck(w.io, "%s b%d h%d final_state" % (name, b, h))
    chk.add(fs[b, h].double().cpu().numpy(), S[0, 0])
    _STATS.setdefault(name, {})[(b, h)] = {"out": so, "final_state": chk.finish()}


def test_ablation_overflow_count_at_full_size():
    # the 1m workload's inputs through the unbounded gate: the GPU's count of non-finite
    # Gamma-scaled diagonal-tile key operands against the CPU predictor over every head and token
    w, inp, out, fs, counts = _run("1m")
    assert counts == [0, 0]
    cnt = torch.zeros(2, dtype=torch.int64, device="cuda")
    o2 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["beta"], g_min=w.g_min, chunk=w.chunk,
                       gate="logsigmoid", counts=cnt)
    torch.cuda.synchronize()
    got = cnt.tolist()
    del o2

    def piece(job):
        b, h, t0 = job
        t1 = min(w.T, t0 + PIECE)  # whole chunks: the predictor's prefix sums restart at each chunk
        a64 = inp["a"][b:b + 1, h:h + 1, t0:t1].to("cpu", torch.float64).numpy()
        k64 = inp["k"][b:b + 1, h:h + 1, t0:t1].to("cpu", torch.float64).numpy()
        return overflow.subtile_operand_overflow(a64, k64, w.g_min, w.chunk, "logsigmoid")

    jobs = [(b, h, t0) for b in range(w.B) for h in range(w.H) for t0 in range(0, w.T, PIECE)]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        res = list(ex.map(piece, jobs))
    pred = sum(r[0] for r in res)
    border = sum(r[1] for r in res)
    _say("ABLATION 1m operands: gpu %d predicted %d borderline %d; non-finite outputs %d of %d; bounded %s" % (
        got[0], pred, border, got[1], w.B * w.H * w.T * w.dv, counts))
    assert pred > 0
    assert abs(got[0] - pred) <= border
    assert got[1] > 0
