"""The C ABI on a machine without a GPU: the library loads, exports every
function include/kda.h declares, sizes the workspace, and rejects bad
arguments with the documented status codes before launching anything."""
import ctypes
import os
import re

import pytest
import torch

import chunked_gated_linear_bounded_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_CHUNK, E_GMIN, E_WS, E_HIP, E_ALIGN, E_MODE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
E_SCRATCH = -10


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    L = kda.lib()
    names = _declared_functions()
    assert {"kda_abi_version", "kda_status_string", "kda_chunk_fwd_workspace_bytes",
            "kda_gate_cumsum", "kda_chunk_fwd", "kda_chunk_fwd_ex", "kda_chunk_intra", "kda_chunk_state",
            "kda_decode_step", "kda_chunk_fwd_varlen", "kda_chunk_fwd_varlen_workspace_bytes",
            "kda_chunk_fwd_lowrank", "kda_chunk_bwd", "kda_chunk_bwd_workspace_bytes",
            "kda_chunk_fwd_noalloc"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings():
    assert kda.abi_version() == 8
    for st in (OK, E_NULL, E_SHAPE, E_DTYPE, E_CHUNK, E_GMIN, E_WS, E_HIP, E_ALIGN, E_MODE, E_SCRATCH):
        s = kda.status_string(st)
        assert s and s != "unknown status"
    assert kda.status_string(12345) == "unknown status"


def test_workspace_bytes():
    # per (batch, head, chunk) record at chunk 64, dk = dv = 128, bf16 I/O (fp16 operand blocks):
    # W^T, Qbar^T, K^ as 32 16-bit tiles each (512 B) + 128 float gammas + 4 int exponents, then for
    # each of the 8 value slices 4 int exponents and U~, Oi^T as 4 fp16 tiles each
    rec = 3 * 32 * 512 + 128 * 4 + 16 + 8 * (16 + 2 * 4 * 512)
    rec = (rec + 255) // 256 * 256
    # 32 heads x 8 value slices fill the 256 compute units: the per-slice state stage, records alone
    assert kda.workspace_bytes(1, 32, 65536, 128, 128, 64, torch.bfloat16) == 32 * 1024 * rec
    # 16 heads: the segmented stage walks each head's 4096 chunks as 16 segments (256 work-groups),
    # per head 16 state slots and 15 transition slots, 128 x 128 float32 each
    seg = 16 * (16 + 15) * 128 * 128 * 4
    assert kda.workspace_bytes(1, 16, 262144, 128, 128, 64, torch.bfloat16) == 16 * 4096 * rec + seg
    # 256 or more heads: the segmented stage with one segment, the records alone
    assert kda.workspace_bytes(4, 64, 8192, 128, 128, 64, torch.bfloat16) == 4 * 64 * 128 * rec
    # fp32 records of 64-token chunks at d = 128 do not fit the segmented stage's ring twice
    L = 3 * 32 * 1024 + 128 * 4 + 16 + 8 * (16 + 2 * 4 * 1024)
    L = (L + 255) // 256 * 256
    assert kda.workspace_bytes(1, 32, 65536, 128, 128, 64, torch.float32) == 32 * 1024 * L
    assert kda.workspace_bytes(1, 2, 256, 64, 64, 16, torch.float32) > 0
    assert kda.workspace_bytes(1, 2, 0, 64, 64, 16, torch.float32) == 0
    assert kda.workspace_bytes(1, 2, 100, 64, 64, 16, torch.float32) == 0   # T % chunk != 0
    assert kda.workspace_bytes(1, 2, 256, 96, 64, 16, torch.float32) == 0   # dk unsupported


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation first


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, beta=FAKE, g_min=-5.0, chunk=64, B=1, H=2, T=128, dk=128, dv=128,
             io=0, out=FAKE, fs=None, ws=FAKE, wsb=1 << 40, stream=None)
    a.update(kw)
    return kda.lib().kda_chunk_fwd(a["q"], a["k"], a["v"], a["a"], a["beta"], a["g_min"], a["chunk"], a["B"],
                                   a["H"], a["T"], a["dk"], a["dv"], a["io"], a["out"], a["fs"], a["ws"],
                                   a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_NULL), (dict(beta=None), E_NULL), (dict(out=None), E_NULL),
    (dict(io=7), E_DTYPE),
    (dict(chunk=48), E_CHUNK), (dict(chunk=128), E_CHUNK),
    (dict(B=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(T=-64), E_SHAPE), (dict(T=100), E_SHAPE),
    (dict(dk=96), E_SHAPE), (dict(dv=256), E_SHAPE), (dict(H=70000), E_SHAPE), (dict(B=70000, T=64), E_SHAPE),
    (dict(g_min=0.0), E_GMIN), (dict(g_min=1.0), E_GMIN), (dict(g_min=-6.0), E_GMIN),
    (dict(g_min=-5.001), E_GMIN), (dict(g_min=-5.6), E_GMIN),
    (dict(g_min=float("nan")), E_GMIN), (dict(g_min=float("-inf")), E_GMIN),
    (dict(ws=None), E_WS), (dict(wsb=1000), E_WS),
    (dict(q=FAKE + 8), E_ALIGN), (dict(out=FAKE + 4), E_ALIGN), (dict(beta=FAKE + 1), E_ALIGN),
    (dict(ws=FAKE + 8), E_ALIGN), (dict(fs=FAKE + 4), E_ALIGN),
])
def test_validation_codes(kw, want):
    assert _fwd(**kw) == want


def test_validation_ex_and_gate():
    L = kda.lib()
    args = [FAKE] * 5 + [-5.0, 64, 1, 2, 128, 128, 128, 0, FAKE, None, FAKE, 1 << 40, None]
    assert L.kda_chunk_fwd_ex(*args, 5, None, None) == E_MODE
    # the ablation mode ignores g_min (it must not be rejected for it) -> fails later on the workspace
    args2 = list(args)
    args2[5] = 3.0
    args2[16] = 10
    assert L.kda_chunk_fwd_ex(*args2, 1, None, None) == E_WS
    assert L.kda_chunk_fwd_ex(*args2, 0, None, None) == E_GMIN
    assert L.kda_chunk_fwd_ex(*args, 0, FAKE + 4, None) == E_ALIGN
    assert L.kda_chunk_fwd_ex(*args, 0, None, FAKE + 4) == E_ALIGN  # initial_state: 16-byte aligned
    assert L.kda_gate_cumsum(None, -5.0, 64, 1, 2, 128, 128, 0, 0, FAKE, None) == E_NULL
    assert L.kda_gate_cumsum(FAKE, -5.0, 64, 1, 2, 100, 128, 0, 0, FAKE, None) == E_SHAPE
    assert L.kda_gate_cumsum(FAKE, 0.5, 64, 1, 2, 128, 128, 0, 0, FAKE, None) == E_GMIN
    assert L.kda_gate_cumsum(FAKE, -5.0, 64, 1, 2, 128, 128, 0, 3, FAKE, None) == E_MODE
    assert L.kda_gate_cumsum(FAKE + 2, -5.0, 64, 1, 2, 128, 128, 0, 0, FAKE, None) == E_ALIGN
    # empty sequence with no final state: nothing to do, no HIP call
    assert _fwd(T=0, ws=None, wsb=0) == OK
    assert _fwd(T=0, q=None, k=None, v=None, a=None, beta=None, out=None, ws=None, wsb=0) == OK
    assert _fwd(T=64, q=None, ws=None, wsb=0) == E_NULL
    assert L.kda_gate_cumsum(FAKE, -5.0, 64, 1, 2, 0, 128, 0, 0, FAKE, None) == OK


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_NULL), (dict(state=None), E_NULL), (dict(out=None), E_NULL),
    (dict(io=3), E_DTYPE), (dict(B=0), E_SHAPE), (dict(dk=32), E_SHAPE), (dict(dv=96), E_SHAPE),
    (dict(g_min=0.0), E_GMIN), (dict(mode=2), E_MODE),
    (dict(state=FAKE + 4), E_ALIGN), (dict(k=FAKE + 2), E_ALIGN), (dict(beta=FAKE + 1), E_ALIGN),
])
def test_decode_validation(kw, want):
    a = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, beta=FAKE, g_min=-5.0, B=1, H=2, dk=128, dv=128, io=0, mode=0,
             state=FAKE, out=FAKE)
    a.update(kw)
    st = kda.lib().kda_decode_step(a["q"], a["k"], a["v"], a["a"], a["beta"], a["g_min"], a["B"], a["H"], a["dk"],
                                   a["dv"], a["io"], a["mode"], a["state"], a["out"], None)
    assert st == want


def test_binding_rejects_host_tensors():
    x = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        kda.chunk_fwd(x, x, x, x, torch.zeros(1, 1, 64), chunk=16)
    with pytest.raises(ValueError):
        kda.gate_cumsum(x, chunk=16)
    with pytest.raises(ValueError):
        kda.decode_step(x[:, :, 0], x[:, :, 0], x[:, :, 0], x[:, :, 0], torch.zeros(1, 1), torch.zeros(1, 1, 64, 64))
    with pytest.raises(ValueError):
        kda.chunk_fwd_varlen(x[0], x[0], x[0], x[0], torch.zeros(1, 64), torch.zeros(2, dtype=torch.int32))


def test_varlen_workspace_bytes():
    # records for T / chunk + N chunks per head (each document may end in a short chunk), then the
    # plan tables: a {token, rows, document, flags} entry per chunk, N + 1 boundaries, N + 1 chunk
    # offsets and R + 1 run boundaries (R = enough runs to give 256 walks over heads and slices, at
    # most N)
    rec = kda.workspace_bytes(1, 1, 64, 128, 128, 64, torch.bfloat16)
    N, H, T = 76, 32, 65536
    nc = T // 64 + N
    assert kda.varlen_workspace_bytes(N, H, T, 128, 128, 64, torch.bfloat16) == \
        H * nc * rec + 16 * nc + 8 * (N + 1) + 4 * (1 + 1)
    rec2 = kda.workspace_bytes(1, 1, 16, 64, 64, 16, torch.float32)
    assert kda.varlen_workspace_bytes(5, 2, 100, 64, 64, 16, torch.float32) == \
        2 * (100 // 16 + 5) * rec2 + 16 * (100 // 16 + 5) + 8 * 6 + 4 * (5 + 1)  # R = min(5, 256 / 8)
    assert kda.varlen_workspace_bytes(3, 2, 100, 64, 64, 16, torch.float32) > 0   # T need not divide by chunk
    assert kda.varlen_workspace_bytes(0, 2, 100, 64, 64, 16, torch.float32) == 0  # no document
    assert kda.varlen_workspace_bytes(3, 2, 100, 96, 64, 16, torch.float32) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_NULL), (dict(cu=None), E_NULL), (dict(ws=None), E_NULL), (dict(out=None), E_NULL),
    (dict(io=2), E_DTYPE), (dict(chunk=8), E_CHUNK), (dict(N=0), E_SHAPE), (dict(H=0), E_SHAPE),
    (dict(T=-1), E_SHAPE), (dict(dk=32), E_SHAPE), (dict(N=1 << 30), E_SHAPE),
    (dict(g_min=-7.0), E_GMIN), (dict(mode=4), E_MODE),
    (dict(cu=FAKE + 2), E_ALIGN), (dict(q=FAKE + 8), E_ALIGN), (dict(fs=FAKE + 8), E_ALIGN),
    (dict(s0=FAKE + 4), E_ALIGN), (dict(wsb=100), E_WS),
])
def test_varlen_validation(kw, want):
    a = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, beta=FAKE, g_min=-5.0, chunk=64, cu=FAKE, N=3, H=2, T=100, dk=128,
             dv=128, io=0, out=FAKE, fs=None, ws=FAKE, wsb=1 << 40, mode=0, s0=None)
    a.update(kw)
    st = kda.lib().kda_chunk_fwd_varlen(a["q"], a["k"], a["v"], a["a"], a["beta"], a["g_min"], a["chunk"], a["cu"],
                                        a["N"], a["H"], a["T"], a["dk"], a["dv"], a["io"], a["out"], a["fs"], a["ws"],
                                        a["wsb"], None, a["mode"], None, a["s0"])
    assert st == want


@pytest.mark.parametrize("kw,want", [
    (dict(h=None), E_NULL), (dict(z=None), E_NULL), (dict(A=None), E_NULL), (dict(q=None), E_NULL),
    (dict(rank=0), E_SHAPE), (dict(rank=8), E_SHAPE), (dict(rank=48), E_SHAPE), (dict(rank=256), E_SHAPE),
    (dict(T=100), E_SHAPE), (dict(io=5), E_DTYPE), (dict(g_min=-9.0), E_GMIN), (dict(mode=3), E_MODE),
    (dict(h=FAKE + 8), E_ALIGN), (dict(z=FAKE + 4), E_ALIGN), (dict(A=FAKE + 2), E_ALIGN), (dict(wsb=64), E_WS),
    (dict(T=0, rank=24), E_SHAPE),
])
def test_lowrank_validation(kw, want):
    a = dict(q=FAKE, k=FAKE, v=FAKE, h=FAKE, z=FAKE, A=FAKE, beta=FAKE, g_min=-5.0, chunk=64, B=1, H=2, T=128,
             dk=128, dv=128, rank=32, io=0, out=FAKE, fs=None, ws=FAKE, wsb=1 << 40, mode=0)
    a.update(kw)
    st = kda.lib().kda_chunk_fwd_lowrank(a["q"], a["k"], a["v"], a["h"], a["z"], a["A"], a["beta"], a["g_min"],
                                         a["chunk"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["rank"], a["io"],
                                         a["out"], a["fs"], a["ws"], a["wsb"], None, a["mode"], None, None)
    assert st == want


def test_bwd_workspace_bytes():
    # the 16-token chunk records plus two float32 states (dk x dv) per 16-token chunk and head
    rec = kda.workspace_bytes(1, 1, 16, 128, 128, 16, torch.bfloat16)
    n = 2 * 16 * (4096 // 16)
    assert kda.bwd_workspace_bytes(2, 16, 4096, 128, 128, torch.bfloat16) == n * (rec + 2 * 128 * 128 * 4)
    assert kda.bwd_workspace_bytes(1, 2, 40, 64, 64, torch.float32) == 0  # T % 16
    assert kda.bwd_workspace_bytes(1, 2, 0, 64, 64, torch.float32) == 0


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), E_NULL), (dict(dout=None), E_NULL), (dict(dq=None), E_NULL), (dict(dbeta=None), E_NULL),
    (dict(T=40), E_SHAPE), (dict(dk=96), E_SHAPE), (dict(B=0), E_SHAPE), (dict(io=2), E_DTYPE),
    (dict(B=300, H=300), E_SHAPE),
    (dict(g_min=0.5), E_GMIN), (dict(mode=7), E_MODE), (dict(dout=FAKE + 8), E_ALIGN),
    (dict(dq=FAKE + 4), E_ALIGN), (dict(s0=FAKE + 4), E_ALIGN), (dict(ws=None), E_WS), (dict(wsb=99), E_WS),
])
def test_bwd_validation(kw, want):
    a = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, beta=FAKE, g_min=-5.0, B=1, H=2, T=64, dk=128, dv=128, io=0, mode=0,
             s0=None, dout=FAKE, dF=None, dq=FAKE, dk_=FAKE, dv_=FAKE, da=FAKE, dbeta=FAKE, dS0=None, ws=FAKE,
             wsb=1 << 40)
    a.update(kw)
    st = kda.lib().kda_chunk_bwd(a["q"], a["k"], a["v"], a["a"], a["beta"], a["g_min"], a["B"], a["H"], a["T"],
                                 a["dk"], a["dv"], a["io"], a["mode"], a["s0"], a["dout"], a["dF"], a["dq"], a["dk_"],
                                 a["dv_"], a["da"], a["dbeta"], a["dS0"], a["ws"], a["wsb"], None)
    assert st == want


def test_lowest_g_min_is_the_pages_constant(golden_dir):
    # the header's most negative accepted g_min is the constant the pages fix (below it the
    # shrunk row operands of a 16-token tile reach the subnormal range), and the ABI accepts it
    import json
    import re
    hdr = open(os.path.join(os.path.dirname(golden_dir), "..", "include", "kda.h")).read()
    lowest = float(re.search(r"#define KDA_G_MIN_LOWEST \((-?[0-9.]+)f\)", hdr).group(1))
    pages = json.load(open(os.path.join(golden_dir, "pages_constants.json")))
    assert lowest == pages["g_min"] == -5.0
    span = 15 * abs(lowest)
    assert span == pages["max_diagonal_exponent"]
    assert span + 12 < pages["ln_bf16_max"] and -span - 12 > pages["ln_bf16_min_normal"]
    # accepted: validation gets past g_min and stops at the (too small) workspace, before any launch
    assert _fwd(g_min=lowest, wsb=1000) == E_WS
    assert _fwd(g_min=lowest - 0.001, wsb=1000) == E_GMIN



def _noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, a=FAKE, beta=FAKE, g_min=-5.0, chunk=64, B=1, H=2, T=256, dk=128, dv=128,
             io=0, out=FAKE, fs=None, stream=None, mode=0, counts=None, init=None)
    a.update(kw)
    return kda.lib().kda_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["a"], a["beta"], a["g_min"], a["chunk"], a["B"],
                                           a["H"], a["T"], a["dk"], a["dv"], a["io"], a["out"], a["fs"], a["stream"],
                                           a["mode"], a["counts"], a["init"])


def test_noalloc_validation():
    # the same checks as kda_chunk_fwd_ex, and the size limit of the static scratch, all before any HIP call
    assert _noalloc(q=None) == E_NULL
    assert _noalloc(out=None) == E_NULL
    assert _noalloc(T=100) == E_SHAPE
    assert _noalloc(chunk=48) == E_CHUNK
    assert _noalloc(io=5) == E_DTYPE
    assert _noalloc(g_min=-6.0) == E_GMIN
    assert _noalloc(mode=3) == E_MODE
    assert _noalloc(out=FAKE + 8) == E_ALIGN
    # one 64-token chunk record of every head must fit in 128 MiB: 1,600 heads do, 1,700 do not;
    # without a final_state the 64 KiB state of every head has to fit beside them
    rec = kda.workspace_bytes(1, 1, 64, 128, 128, 64, torch.bfloat16)
    limit = 128 << 20
    fits = limit // rec
    assert _noalloc(H=fits + 1, fs=FAKE) == E_SCRATCH
    with_state = limit // (rec + 128 * 128 * 4)
    assert _noalloc(H=with_state + 1) == E_SCRATCH
    assert with_state < fits
