"""Pins of the oracle against facts fixed by the pages and by mathematics.

None of these compares the oracle with a retyped copy of itself: each check uses
a value derived by hand, a closed form of a special case, an independent
formulation (brute-force products of dense transition matrices, the quadratic
form of decayed linear attention, the chunk-parallel WY/UT form), or an
invariant of the definition.  A dropped term, a wrong sign, a transposed state
or a shifted cumulative sum fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import native, overflow, reference

RNG = np.random.default_rng(12345)


def _rand_case(B, H, T, dk, dv, rng, a_sigma=1.0, norm=True, beta=None):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if norm:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    a = rng.standard_normal((B, H, T, dk)) * a_sigma
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T)))) if beta is None else np.full((B, H, T), beta)
    return q, k, v, a, b


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _parse(x):
    return float(x)  # handles "inf", "-inf", "0"


# ---------------------------------------------------------------- hand-derived case
@pytest.mark.parametrize("case", ["bounded", "logsigmoid"])
@pytest.mark.parametrize("impl", ["c", "numpy", "chunked1", "chunked2", "brute"])
def test_hand_derived_delta_rule(golden_dir, case, impl):
    gd = _golden(golden_dir, "hand_delta_rule.json")
    tok = gd["tokens"]
    c = gd["cases"][case]
    k = np.array(tok["k"])[None, None]
    v = np.array(tok["v"])[None, None]
    q = np.array(tok["q"])[None, None]
    beta = np.array(tok["beta"])[None, None]
    a = np.array([[_parse(x) for x in row] for row in c["a"]])[None, None]
    d = math.exp(-2.5) if case == "bounded" else 0.5
    g_min = c.get("g_min", -5.0)
    env = {"d": d}
    want_out = np.array([[eval(x, {}, env) for x in row] for row in gd["out_in_terms_of_d"]])
    want_fin = np.array([[eval(x, {}, env) for x in row] for row in gd["final_state_in_terms_of_d"]])
    with np.errstate(over="ignore", invalid="ignore"):
        if impl == "c":
            out, fin = native.recurrent(q, k, v, a, beta, g_min, gate=case)
        elif impl == "numpy":
            out, fin = reference.recurrent(q, k, v, a, beta, g_min, case)
        elif impl.startswith("chunked"):
            out, fin = reference.chunked(q, k, v, a, beta, int(impl[-1]), g_min, case, decay_ref="pairwise")
        else:
            out, fin = reference.brute_force(q, k, v, a, beta, g_min, case)
    np.testing.assert_allclose(out[0, 0], want_out, atol=1e-14, rtol=0)
    np.testing.assert_allclose(fin[0, 0], want_fin, atol=1e-14, rtol=0)


# ---------------------------------------------------------------- the gate
def test_gate_values():
    # g_min * sigmoid(0) = g_min / 2 ; sigmoid(+-inf) = 1, 0
    assert reference.gate(np.array(0.0)) == -2.5
    assert reference.gate(np.array(np.inf)) == -5.0
    assert reference.gate(np.array(-np.inf)) == 0.0
    a = RNG.standard_normal(10000) * 50
    g = reference.gate(a)
    assert g.min() >= -5.0 and g.max() <= 0.0
    # log sigmoid: -ln 2 at 0, exact for large |a| where the naive form fails
    assert abs(reference.gate(np.array(0.0), mode="logsigmoid") + math.log(2.0)) < 1e-16
    assert reference.gate(np.array(-1000.0), mode="logsigmoid") == -1000.0
    assert reference.gate(np.array(1000.0), mode="logsigmoid") == 0.0
    a = np.linspace(-30, 30, 601)
    naive = np.log(1.0 / (1.0 + np.exp(-a)))
    np.testing.assert_allclose(reference.gate(a, mode="logsigmoid"), naive, rtol=1e-12, atol=1e-15)


def test_pages_constants(golden_dir):
    gc = _golden(golden_dir, "pages_constants.json")
    bmax = float(torch.finfo(torch.bfloat16).max)
    btiny = float(torch.finfo(torch.bfloat16).tiny)
    assert abs(math.log(bmax) - gc["ln_bf16_max"]) < 1e-12
    assert abs(math.log(btiny) - gc["ln_bf16_min_normal"]) < 1e-12
    span = (gc["safe_tile_tokens"] - 1) * abs(gc["g_min"])
    assert span == gc["max_diagonal_exponent"]
    assert span < gc["ln_bf16_max"] and -span > gc["ln_bf16_min_normal"]
    assert reference.G_MIN == gc["g_min"] and reference.SUBTILE == gc["safe_tile_tokens"]


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
@pytest.mark.parametrize("with_s0", [False, True])
def test_brute_force(gate, with_s0):
    rng = np.random.default_rng(7 + with_s0)
    q, k, v, a, b = _rand_case(1, 2, 9, 5, 4, rng, a_sigma=2.0)
    S0 = rng.standard_normal((1, 2, 4, 5)) if with_s0 else None
    out_c, fin_c = native.recurrent(q, k, v, a, b, -5.0, gate=gate, S0=S0)
    out_b, fin_b = reference.brute_force(q, k, v, a, b, -5.0, gate, S0=S0)
    np.testing.assert_allclose(out_c, out_b, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(fin_c, fin_b, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- special cases
def test_scalar_full_erase():
    # dk = dv = 1, k = +-1, beta = 1: S_{t-1} e^g (1 - k^2) = 0, so S_t = v_t k_t, o_t = v_t k_t q_t
    rng = np.random.default_rng(3)
    T = 40
    k = np.sign(rng.standard_normal((1, 1, T, 1)))
    q, v, a = (rng.standard_normal((1, 1, T, 1)) for _ in range(3))
    out, fin = native.recurrent(q, k, v, a, np.ones((1, 1, T)))
    np.testing.assert_allclose(out, v * k * q, atol=1e-15)
    np.testing.assert_allclose(fin[0, 0, 0, 0], v[0, 0, -1, 0] * k[0, 0, -1, 0], atol=1e-15)


@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
def test_erase_free_is_decayed_linear_attention(gate):
    # Without the erase term the recurrence is plain decayed linear attention,
    # whose quadratic form needs no state at all.
    rng = np.random.default_rng(11)
    q, k, v, a, b = _rand_case(2, 2, 30, 6, 5, rng, a_sigma=2.0)
    S0 = rng.standard_normal((2, 2, 5, 6))
    out, _ = native.recurrent(q, k, v, a, b, -5.0, gate=gate, erase=False, S0=S0)
    want = reference.decayed_linear_attention(q, k, v, a, b, -5.0, gate, S0=S0)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)


def test_no_decay_no_erase_is_cumulative_sum():
    # g = 0 (a = -inf under the bounded gate), beta = 1, no erase:
    # S_t = sum_{s<=t} v_s k_s^T,  o_t = sum_{s<=t} (k_s . q_t) v_s
    rng = np.random.default_rng(5)
    q, k, v, _, _ = _rand_case(1, 3, 25, 7, 3, rng, norm=False)
    a = np.full(q.shape, -np.inf)
    with np.errstate(over="ignore"):
        out, fin = native.recurrent(q, k, v, a, np.ones(q.shape[:3]), erase=False)
    kv = np.cumsum(np.einsum("bhti,bhtj->bhtij", v, k), axis=2)
    np.testing.assert_allclose(fin, kv[:, :, -1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, np.einsum("bhtij,bhtj->bhti", kv, q), rtol=1e-11, atol=1e-12)


def test_beta_zero_gives_zero():
    rng = np.random.default_rng(6)
    q, k, v, a, _ = _rand_case(1, 2, 50, 8, 8, rng)
    out, fin = native.recurrent(q, k, v, a, np.zeros(q.shape[:3]))
    assert np.all(out == 0.0) and np.all(fin == 0.0)


@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
def test_delta_rule_retrieval(gate):
    # beta = 1 and |k| = 1: the delta rule stores v_t exactly under k_t, S_t k_t = v_t,
    # whatever the decay; with q = k the output is v.
    rng = np.random.default_rng(8)
    _, k, v, a, _ = _rand_case(1, 2, 64, 16, 12, rng, a_sigma=3.0)
    out, _ = native.recurrent(k, k, v, a, np.ones(k.shape[:3]), -5.0, gate=gate)
    np.testing.assert_allclose(out, v, atol=1e-12)


# ---------------------------------------------------------------- chunk form
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("decay_ref", ["pairwise", "chunk", "subtile"])
def test_chunked_equals_recurrent(chunk, decay_ref):
    rng = np.random.default_rng(chunk)
    T = 3 * chunk + 19  # several chunks and a ragged tail
    q, k, v, a, b = _rand_case(1, 2, T, 16, 8, rng, a_sigma=4.0)
    S0 = rng.standard_normal((1, 2, 8, 16)) * 0.3
    out_c, fin_c = native.recurrent(q, k, v, a, b, S0=S0)
    out_k, fin_k = reference.chunked(q, k, v, a, b, chunk, S0=S0, decay_ref=decay_ref)
    scale = np.sqrt(np.mean(out_c ** 2))
    assert np.max(np.abs(out_k - out_c)) <= 1e-12 * max(scale, 1.0)
    assert np.max(np.abs(fin_k - fin_c)) <= 1e-12 * max(np.sqrt(np.mean(fin_c ** 2)), 1.0)


def test_c_and_numpy_transcriptions_agree():
    rng = np.random.default_rng(21)
    q, k, v, a, b = _rand_case(2, 3, 120, 32, 24, rng, a_sigma=2.0)
    for gate in ("bounded", "logsigmoid"):
        o1, f1 = native.recurrent(q, k, v, a, b, -5.0, gate=gate)
        o2, f2 = reference.recurrent(q, k, v, a, b, -5.0, gate)
        np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(f1, f2, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants
def test_linear_in_v_causal_and_head_independent():
    rng = np.random.default_rng(31)
    q, k, v, a, b = _rand_case(1, 2, 80, 8, 6, rng, a_sigma=2.0)
    v2 = rng.standard_normal(v.shape)
    o1, _ = native.recurrent(q, k, v, a, b)
    o2, _ = native.recurrent(q, k, v2, a, b)
    o3, _ = native.recurrent(q, k, 2.0 * v - 3.0 * v2, a, b)
    np.testing.assert_allclose(o3, 2.0 * o1 - 3.0 * o2, rtol=1e-11, atol=1e-12)
    # causality: perturbing token 50 leaves outputs before it bitwise unchanged
    kp = k.copy()
    kp[:, :, 50] = -kp[:, :, 50]
    o4, _ = native.recurrent(q, kp, v, a, b)
    assert np.array_equal(o4[:, :, :50], o1[:, :, :50])
    assert not np.allclose(o4[:, :, 50:], o1[:, :, 50:])
    # heads are independent: head 1 alone gives the same result
    o5, _ = native.recurrent(q[:, 1:], k[:, 1:], v[:, 1:], a[:, 1:], b[:, 1:])
    assert np.array_equal(o5[:, 0], o1[:, 1])


# ---------------------------------------------------------------- the bound (P8) and the ablation predictor (P9)
def test_bounded_gate_keeps_subtile_exponent_within_bf16():
    rng = np.random.default_rng(41)
    a = rng.standard_normal((1, 2, 1024, 32)) * 40.0   # drive many gates to g_min
    span = overflow.subtile_spans(a, -5.0, 64, "bounded")
    assert span <= 15 * 5.0 + 1e-9 and span < math.log(float(torch.finfo(torch.bfloat16).max))
    k = rng.standard_normal(a.shape)
    assert overflow.subtile_operand_overflow(a, k, -5.0, 64, "bounded") == (0, 0)
    # the same gates without the bound exceed the range inside a 16-token tile
    assert overflow.subtile_spans(a, -5.0, 64, "logsigmoid") > 88.72
    assert overflow.subtile_operand_overflow(a, k, -5.0, 64, "logsigmoid")[0] > 0
    # and a whole-64-chunk reference overflows even with the bound
    assert overflow.whole_chunk_inverse_overflow(a, k, -5.0, 64, "bounded") > 0


def test_whole_chunk_inverse_overflow_exact_counts():
    # k = 1 and a constant gate g: referenced to the chunk start, the inverse decay of row s of a
    # 64-token chunk is 2^(|g| log2(e) (s + 1)) (inclusive prefix sum), which overflows bf16 from the
    # first row whose exponent reaches the bf16 threshold (~127.997); |k| = 2^10 lowers that row by
    # ten exponent units.
    T = 256
    k = np.ones((1, 1, T, 1))
    a = np.full((1, 1, T, 1), 50.0)  # sigmoid(50) is 1 in float64: g = -5, 7.2135 per row -> rows 17..63
    assert overflow.whole_chunk_inverse_overflow(a, k, -5.0, 64, "bounded") == 47 * (T // 64)
    a0 = np.zeros((1, 1, T, 1))  # g = -2.5, 3.6067 per row -> rows 35..63
    assert overflow.whole_chunk_inverse_overflow(a0, k, -5.0, 64, "bounded") == 29 * (T // 64)
    k10 = np.full((1, 1, T, 1), 1024.0)  # exponent + 10 -> rows 16..63
    assert overflow.whole_chunk_inverse_overflow(a, k10, -5.0, 64, "bounded") == 48 * (T // 64)


def test_overflow_predictor_exact_counts():
    # k = 1, constant gate.  Inside a 16-token tile the operand for offset j is
    # 2^(j*|g|*log2 e); it is non-finite in bf16 exactly when that exponent
    # reaches the bf16 overflow threshold (~127.997).
    T = 256
    k = np.ones((1, 1, T, 1))
    # unbounded gate at a = -20: |g| = 20 + 2e-9 -> 28.85 per step -> offsets 5..15 overflow
    a = np.full((1, 1, T, 1), -20.0)
    assert overflow.subtile_operand_overflow(a, k, -5.0, 64, "logsigmoid") == (11 * T // 16, 0)
    # bounded gate pinned at g_min = -5: 7.21 per step, at most 108.2 -> none
    a = np.full((1, 1, T, 1), np.inf)
    assert overflow.subtile_operand_overflow(a, k, -5.0, 64, "bounded") == (0, 0)
    # a bound of -6 is not enough: 8.656 per step -> offset 15 (129.8) overflows
    assert overflow.subtile_operand_overflow(a, k, -6.0, 64, "bounded") == (T // 16, 0)


def test_overflow_predictor_counts_per_head_and_ragged_tail():
    # the same closed form with a different constant gate per (b, h) slab, so the counts add up
    # over the batch and head axes: |g| = 30, 20, 10 per step overflow from offset 3, 5, 9 on
    # (13, 11, 7 of 16 per tile); the bounded gate never.  T = 264 ends in a partial tile of 8
    # tokens (and a partial chunk), where offsets 5..7 of the |g| = 20 slab overflow.
    k = np.ones((2, 3, 256, 1))
    a = np.empty_like(k)
    for (b, h), x in zip(np.ndindex(2, 3), (-30.0, -20.0, -10.0, -20.0, -30.0, -10.0)):
        a[b, h] = x
    assert overflow.subtile_operand_overflow(a, k, -5.0, 64, "logsigmoid") == (16 * 2 * (13 + 11 + 7), 0)
    a = np.full((1, 1, 264, 1), -20.0)
    assert overflow.subtile_operand_overflow(a, np.ones_like(a), -5.0, 64, "logsigmoid") == (16 * 11 + 3, 0)


# ---------------------------------------------------------------- the initial state
@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
def test_beta_zero_state_only_decays(gate):
    """beta = 0: nothing is written or erased, so S_t = S0 diag(e^{G_t}) with G_t the running sum
    of the gate from the first token, and o_t = S_t q_t (closed form)."""
    rng = np.random.default_rng(31)
    q, k, v, a, _ = _rand_case(1, 2, 24, 6, 5, rng, a_sigma=2.0)
    b = np.zeros((1, 2, 24))
    S0 = rng.standard_normal((1, 2, 5, 6))
    out, fin = native.recurrent(q, k, v, a, b, -5.0, gate=gate, S0=S0)
    g = -5.0 / (1.0 + np.exp(-a)) if gate == "bounded" else -np.logaddexp(0.0, -a)
    G = np.cumsum(g, axis=2)
    want = np.einsum("bhij,bhtj->bhti", S0, np.exp(G) * q)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-14)
    assert np.allclose(fin, S0 * np.exp(G[:, :, -1, None, :]), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("split", [1, 7, 16])
def test_sequence_split_continues_from_the_final_state(split):
    """The state summarises the past: running tokens [0, T1) and then [T1, T) from its final state
    gives the single run's outputs and final state (both the C and the NumPy form)."""
    rng = np.random.default_rng(32 + split)
    q, k, v, a, b = _rand_case(2, 2, 32, 6, 5, rng)
    out, fin = native.recurrent(q, k, v, a, b)
    s1 = slice(0, split)
    s2 = slice(split, 32)
    o1, f1 = native.recurrent(q[:, :, s1], k[:, :, s1], v[:, :, s1], a[:, :, s1], b[:, :, s1])
    o2, f2 = reference.recurrent(q[:, :, s2], k[:, :, s2], v[:, :, s2], a[:, :, s2], b[:, :, s2], S0=f1)
    assert np.allclose(np.concatenate([o1, o2], axis=2), out, rtol=1e-12, atol=1e-13)
    assert np.allclose(f2, fin, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- packed documents
def _packed(lengths, rng, H=2, dk=6, dv=5):
    T = int(sum(lengths))
    q, k, v, a, b = _rand_case(1, H, T, dk, dv, rng, a_sigma=2.0)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return q[0], k[0], v[0], a[0], b[0], cu


def test_packed_first_token_of_every_document():
    """From a zero state one token leaves S_1 = beta v k^T (the decayed zero state adds nothing), so
    the first output of every document is beta (k . q) v and a one-token document ends in
    beta v k^T (closed form): a state carried across a boundary, or a boundary off by one,
    breaks it."""
    rng = np.random.default_rng(41)
    lengths = [5, 1, 7, 3, 1, 9]
    q, k, v, a, b, cu = _packed(lengths, rng)
    out, fin = native.recurrent_varlen(q, k, v, a, b, cu)
    for i, s in enumerate(cu[:-1]):
        kq = np.sum(k[:, s] * q[:, s], axis=-1)
        assert np.allclose(out[:, s], (b[:, s] * kq)[:, None] * v[:, s], rtol=1e-13, atol=1e-15)
        if lengths[i] == 1:
            assert np.allclose(fin[i], b[:, s, None, None] * v[:, s, :, None] * k[:, s, None, :], rtol=1e-13,
                               atol=1e-15)


def test_packed_documents_do_not_interact():
    """Changing one document's tokens changes nothing in the others, and reordering the documents
    moves each one's outputs and final state along with it unchanged."""
    rng = np.random.default_rng(42)
    lengths = [6, 11, 4]
    q, k, v, a, b, cu = _packed(lengths, rng)
    out, fin = native.recurrent_varlen(q, k, v, a, b, cu)
    q2, v2, a2 = q.copy(), v.copy(), a.copy()
    q2[:, cu[1]:cu[2]] += 1.0
    v2[:, cu[1]:cu[2]] *= -3.0
    a2[:, cu[1]:cu[2]] += 2.0
    out2, fin2 = native.recurrent_varlen(q2, k, v2, a2, b, cu)
    for i in (0, 2):
        assert np.array_equal(out2[:, cu[i]:cu[i + 1]], out[:, cu[i]:cu[i + 1]])
        assert np.array_equal(fin2[i], fin[i])
    assert not np.allclose(out2[:, cu[1]:cu[2]], out[:, cu[1]:cu[2]])
    order = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in order])
    cu3 = np.concatenate([[0], np.cumsum([lengths[i] for i in order])])
    out3, fin3 = native.recurrent_varlen(q[:, idx], k[:, idx], v[:, idx], a[:, idx], b[:, idx], cu3)
    assert np.allclose(out3, out[:, idx], rtol=1e-13, atol=1e-15)
    assert np.allclose(fin3, fin[order], rtol=1e-13, atol=1e-15)


def test_packed_empty_document_keeps_its_initial_state():
    """A document with no tokens has no outputs and ends in the state it started from; with
    beta = 0 everywhere every document's state only decays from its own initial state
    (closed form S0[i] diag(e^{G}) with G summed over that document alone)."""
    rng = np.random.default_rng(43)
    lengths = [4, 0, 6]
    q, k, v, a, _, cu = _packed(lengths, rng)
    b = np.zeros(q.shape[:2])
    S0 = rng.standard_normal((3, 2, 5, 6))
    out, fin = native.recurrent_varlen(q, k, v, a, b, cu, S0=S0)
    g = -5.0 / (1.0 + np.exp(-a))
    assert np.array_equal(fin[1], S0[1])
    for i in (0, 2):
        G = np.sum(g[:, cu[i]:cu[i + 1]], axis=1)  # [H, dk]
        assert np.allclose(fin[i], S0[i] * np.exp(G)[:, None, :], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- low-rank gate pre-activation
def test_lowrank_preactivation_hand_values():
    """One token, rank 2, two channels, two heads, worked by hand:
    head 0: z = [[3, -1], [0.5, 4]], A = [0, ln 2]:  a = [1*3 + 2*(-1), 2 * (1*0.5 + 2*4)] = [1, 17]
    head 1: z = [[0, 1], [-2, 0]],   A = [ln 3, 0]:   a = [3 * 2, -2]"""
    h = np.array([[[1.0, 2.0]]])
    z = np.array([[[3.0, -1.0], [0.5, 4.0]], [[0.0, 1.0], [-2.0, 0.0]]])
    A = np.array([[0.0, math.log(2.0)], [math.log(3.0), 0.0]])
    a = reference.lowrank_preactivation(h, z, A)
    assert a.shape == (1, 2, 1, 2)
    assert np.allclose(a[0, :, 0], [[1.0, 17.0], [6.0, -2.0]], rtol=1e-15, atol=0)


def test_lowrank_preactivation_special_cases():
    """z = identity (rank = dk) and A = 0 give a = h on every head; scaling z by s and adding
    -ln s to A leaves a unchanged; the factor is shared, so heads with equal z and A agree."""
    rng = np.random.default_rng(44)
    B, T, dk = 2, 5, 8
    h = rng.standard_normal((B, T, dk))
    z = np.broadcast_to(np.eye(dk), (3, dk, dk)).copy()
    a = reference.lowrank_preactivation(h, z, np.zeros((3, dk)))
    for hd in range(3):
        assert np.array_equal(a[:, hd], h)
    R = 4
    h2 = rng.standard_normal((B, T, R))
    z2 = rng.standard_normal((3, dk, R))
    A2 = rng.standard_normal((3, dk))
    a2 = reference.lowrank_preactivation(h2, z2, A2)
    a3 = reference.lowrank_preactivation(h2, z2 * 8.0, A2 - math.log(8.0))
    assert np.allclose(a2, a3, rtol=1e-13, atol=1e-15)
    z2[2] = z2[0]
    A2[2] = A2[0]
    a4 = reference.lowrank_preactivation(h2, z2, A2)
    assert np.array_equal(a4[:, 2], a4[:, 0])


# ---------------------------------------------------------------- gradients (the backward)
def _loss_fd(args, name, loss, h=1e-6):
    x = args[name]
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (loss(**dict(args, **{name: xp})) - loss(**dict(args, **{name: xm}))) / (2 * h)
    return fd


@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
def test_backward_matches_finite_differences(gate):
    """Every gradient of L = sum(dout * out) + sum(dfinal * S_T) against central differences of
    the forward oracle, over 70 tokens (across a 64-token checkpoint block of the adjoint), with
    an initial state."""
    rng = np.random.default_rng(51)
    q, k, v, a, b = _rand_case(1, 2, 70, 3, 2, rng, a_sigma=2.0)
    S0 = rng.standard_normal((1, 2, 2, 3))
    do = rng.standard_normal(v.shape)
    dF = rng.standard_normal(S0.shape)
    g = native.backward(q, k, v, a, b, do, -5.0, gate, S0=S0, dfinal=dF)

    def loss(q, k, v, a, b, S0):
        o, f = native.recurrent(q, k, v, a, b, -5.0, gate=gate, S0=S0)
        return float((o * do).sum() + (f * dF).sum())

    args = dict(q=q, k=k, v=v, a=a, b=b, S0=S0)
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("a", "da"), ("b", "dbeta"), ("S0", "dS0")):
        fd = _loss_fd(args, name, loss)
        assert np.allclose(g[key], fd, rtol=1e-6, atol=1e-8), (name, float(np.abs(g[key] - fd).max()))


def test_backward_single_token_closed_form():
    """One token from S0: S_1 = S0 D (I - beta k k^T) + beta v k^T with D = diag(e^g), so for
    L = dout . (S_1 q):  dv = beta (k . q) dout,  dbeta = (k . q)(v . dout) - (S0 D k . dout)(k . q),
    dq = S_1^T dout,  dS0 = ((dout q^T)(I - beta k k^T)) D  (worked by hand)."""
    rng = np.random.default_rng(52)
    dk, dv = 4, 3
    q, k, v, a, b = _rand_case(1, 1, 1, dk, dv, rng)
    S0 = rng.standard_normal((1, 1, dv, dk))
    do = rng.standard_normal((1, 1, 1, dv))
    g = native.backward(q, k, v, a, b, do, -5.0, "bounded", S0=S0)
    qv, kv, vv, bt, dov = q[0, 0, 0], k[0, 0, 0], v[0, 0, 0], b[0, 0, 0], do[0, 0, 0]
    D = np.diag(np.exp(-5.0 / (1.0 + np.exp(-a[0, 0, 0]))))
    S0m = S0[0, 0]
    E = np.eye(dk) - bt * np.outer(kv, kv)
    S1 = S0m @ D @ E + bt * np.outer(vv, kv)
    kq = kv @ qv
    assert np.allclose(g["dv"][0, 0, 0], bt * kq * dov, rtol=1e-13)
    assert np.allclose(g["dbeta"][0, 0, 0], kq * (vv @ dov) - (S0m @ D @ kv @ dov) * kq, rtol=1e-12)
    assert np.allclose(g["dq"][0, 0, 0], S1.T @ dov, rtol=1e-12)
    assert np.allclose(g["dS0"][0, 0], np.outer(dov, qv) @ E @ D, rtol=1e-12)


def test_backward_zero_incoming_gradient_is_zero():
    rng = np.random.default_rng(53)
    q, k, v, a, b = _rand_case(1, 2, 20, 4, 3, rng)
    g = native.backward(q, k, v, a, b, np.zeros(v.shape), -5.0, "bounded", S0=rng.standard_normal((1, 2, 3, 4)))
    for key in ("dq", "dk", "dv", "da", "dbeta", "dS0"):
        assert not np.any(g[key]), key


@pytest.mark.parametrize("gate", ["bounded", "logsigmoid"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunked_backward_equals_the_adjoint(gate, chunk):
    """The chunk-form backward (the algorithm of the GPU backward) against the hand-written token
    adjoint, 83 tokens (a ragged last chunk), with an initial state and a final-state gradient."""
    rng = np.random.default_rng(54)
    q, k, v, a, b = _rand_case(1, 2, 83, 8, 6, rng, a_sigma=3.0)
    S0 = rng.standard_normal((1, 2, 6, 8))
    do = rng.standard_normal(v.shape)
    dF = rng.standard_normal(S0.shape)
    ref = native.backward(q, k, v, a, b, do, -5.0, gate, S0=S0, dfinal=dF)
    got = reference.chunked_backward(q, k, v, a, b, do, chunk, -5.0, gate, S0=S0, dfinal=dF)
    for key in ref:
        assert np.allclose(got[key], ref[key], rtol=1e-11, atol=1e-12), key
