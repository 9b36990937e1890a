"""Pins of the double-precision oracle against facts fixed independently of it.

Each test checks the oracle (``oracle.forward``, the token-by-token C
recurrence) against something other than itself: a hand-worked example, a
closed form, a brute-force formula of a different shape (explicit matrix
products, plain causal linear attention), an invariant of the operator, or the
independent chunked rewriting in ``oracle.chunked_ref``.  Together they are
chosen so that a dropped term, a wrong sign, a shifted index or a transposed
operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from oracle import chunked_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_problem(seed, B=1, T=37, H=2, dk=8, dv=6, direction="fwd", la_shift=0.5, state_std=0.3):
    w = synth.Workload("pin", B, H, T, dk, dv, "f32", direction, la_shift, state_std, seed)
    return synth.generate(w)


def _unit(x):
    return x / np.maximum(np.linalg.norm(x, axis=-1, keepdims=True), 1e-6)


def test_hand_worked_example():
    """Two tokens worked by hand (tests/golden/hand_worked_2token.json)."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_2token.json")))
    inp, exp = g["inputs"], g["expected"]
    q = np.array(inp["q"], np.float32)[None, :, None, :]
    k = np.array(inp["k"], np.float32)[None, :, None, :]
    v = np.array(inp["v"], np.float32)[None, :, None, :]
    la = np.log(np.array([inp["alpha_fwd"], inp["alpha_rev"]], np.float64)).astype(np.float32)[:, None, :, None]
    bt = np.array([inp["beta_fwd"], inp["beta_rev"]], np.float32)[:, None, :, None]
    # log(1/2) is not exact in fp32: exp(fl(log 0.5)) differs from 0.5 by ~3e-8 relative
    tol = dict(rtol=0, atol=1e-7)
    o, s = oracle.forward(q, k, v, la[:1], bt[:1], None, "fwd")
    np.testing.assert_allclose(o[0, :, 0], exp["out_fwd"], **tol)
    np.testing.assert_allclose(s[0, 0, 0], exp["state_fwd"], **tol)
    o, s = oracle.forward(q, k, v, la[1:], bt[1:], None, "rev")
    np.testing.assert_allclose(o[0, :, 0], exp["out_rev"], **tol)
    np.testing.assert_allclose(s[0, 0, 0], exp["state_rev"], **tol)
    o, s = oracle.forward(q, k, v, la, bt, None, "bi")
    np.testing.assert_allclose(o[0, :, 0], exp["out_bi"], **tol)
    np.testing.assert_allclose(s[0, 0, 0], exp["state_fwd"], **tol)
    np.testing.assert_allclose(s[1, 0, 0], exp["state_rev"], **tol)


def test_no_write_no_decay_keeps_state():
    """beta = 0, a = 1: nothing is written or erased, o_t = S_in q^_t exactly."""
    x = _rand_problem(1)
    la = np.zeros_like(x["log_alpha"])
    bt = np.zeros_like(x["beta"])
    o, s = oracle.forward(x["q"], x["k"], x["v"], la, bt, x["state_in"], "fwd")
    S0 = x["state_in"][0, 0].astype(np.float64)
    qh = _unit(x["q"][0].astype(np.float64))
    ref = np.einsum("hvk,thk->thv", S0, qh)
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-14)
    np.testing.assert_array_equal(s, x["state_in"].astype(np.float64))


def _linear_attention(q, k, v, la, bt):
    """Brute-force gated causal linear attention (no erase), one chain, double."""
    qh, kh = _unit(q.astype(np.float64)), _unit(k.astype(np.float64))
    g = np.cumsum(la.astype(np.float64))
    T = q.shape[0]
    out = np.zeros((T, v.shape[1]))
    for t in range(T):
        for j in range(t + 1):
            out[t] += np.exp(g[t] - g[j]) * bt[j] * (qh[t] @ kh[j]) * v[j]
    return out


def test_small_write_limit_is_linear_attention():
    """a = 1, beta = eps: o_t / eps -> sum_{j<=t} (q^_t . k^_j) v_j (erase is O(eps^2))."""
    x = _rand_problem(2, T=40, state_std=0.0)
    eps = 1e-8
    la = np.zeros_like(x["log_alpha"])
    bt = np.full_like(x["beta"], eps)
    o, _ = oracle.forward(x["q"], x["k"], x["v"], la, bt, None, "fwd")
    for h in range(2):
        ref = _linear_attention(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h], la[0, 0, :, h],
                                np.ones(40))
        np.testing.assert_allclose(o[0, :, h] / np.float32(eps), ref, rtol=1e-5, atol=1e-6)


def test_erase_off_equals_gated_linear_attention():
    """Erase-off mode (S <- aS + beta v k^T) equals brute-force gated linear attention.

    At a = 1, beta = 1 this is plain causal linear attention; the random gates
    also pin where the decay is applied relative to the write.
    """
    x = _rand_problem(3, T=33, state_std=0.0)
    o, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None, "fwd", erase=False)
    for h in range(2):
        ref = _linear_attention(x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h], x["log_alpha"][0, 0, :, h],
                                x["beta"][0, 0, :, h].astype(np.float64))
        np.testing.assert_allclose(o[0, :, h], ref, rtol=0, atol=1e-12)
    ones = np.ones_like(x["beta"])
    o, _ = oracle.forward(x["q"], x["k"], x["v"], np.zeros_like(x["log_alpha"]), ones, None, "fwd", erase=False)
    ref = _linear_attention(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], np.zeros(33), np.ones(33))
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=0, atol=1e-12)


def test_full_write_recalls_value():
    """Unit keys, beta = 1, a = 1: after token t the state maps k^_t exactly to v_t."""
    x = _rand_problem(4, T=12, dk=16, dv=5)
    la = np.zeros_like(x["log_alpha"])
    bt = np.ones_like(x["beta"])
    for t in (0, 1, 5, 11):
        sl = slice(0, t + 1)
        _, s = oracle.forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], la[:, :, sl], bt[:, :, sl],
                              x["state_in"], "fwd")
        for h in range(2):
            kh = _unit(x["k"][0, t, h].astype(np.float64))
            np.testing.assert_allclose(s[0, 0, h] @ kh, x["v"][0, t, h], rtol=0, atol=1e-13)


def test_transition_is_nonexpansive():
    """beta in [0,1], unit keys: eigenvalues of I - beta k k^T are {1, 1-beta}, so with
    v = 0 the state's Frobenius norm never grows (compare the non-expansive inherited
    state of "Video DeltaNet", "Key Contributions" item 2)."""
    rng = np.random.default_rng(0)
    for _ in range(20):
        kk = _unit(rng.standard_normal(9))
        b = rng.uniform()
        M = np.eye(9) - b * np.outer(kk, kk)
        ev = np.sort(np.linalg.eigvalsh(M))
        np.testing.assert_allclose(ev, np.sort(np.r_[1 - b, np.ones(8)]), atol=1e-12)
        # power iteration on M^T M agrees: spectral norm <= 1
        z = rng.standard_normal(9)
        for _ in range(200):
            z = M.T @ (M @ z)
            z /= np.linalg.norm(z)
        assert np.linalg.norm(M @ z) <= 1 + 1e-12
    x = _rand_problem(5, T=30, state_std=1.0)
    v0 = np.zeros_like(x["v"])
    prev = np.linalg.norm(x["state_in"][0, 0, 0])
    for t in range(30):
        sl = slice(0, t + 1)
        _, s = oracle.forward(x["q"][:, sl], x["k"][:, sl], v0[:, sl], x["log_alpha"][:, :, sl],
                              x["beta"][:, :, sl], x["state_in"], "fwd")
        cur = np.linalg.norm(s[0, 0, 0])
        assert cur <= prev * (1 + 1e-14)
        prev = cur


def test_explicit_product_expansion():
    """T <= 16: S_t = S_0 prod A_s + sum_j beta_j v_j k^_j^T prod_{j<s<=t} A_s with
    A_s = a_s (I - beta_s k^_s k^_s^T) formed as explicit dk x dk matrices."""
    x = _rand_problem(6, T=16, dk=7, dv=4)
    o, s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd")
    for h in range(2):
        kh = _unit(x["k"][0, :, h].astype(np.float64))
        qh = _unit(x["q"][0, :, h].astype(np.float64))
        a = np.exp(x["log_alpha"][0, 0, :, h].astype(np.float64))
        b = x["beta"][0, 0, :, h].astype(np.float64)
        v = x["v"][0, :, h].astype(np.float64)
        A = [a[s_] * (np.eye(7) - b[s_] * np.outer(kh[s_], kh[s_])) for s_ in range(16)]
        for t in range(16):
            P = np.eye(7)
            for s_ in range(t + 1):
                P = P @ A[s_]
            St = x["state_in"][0, 0, h].astype(np.float64) @ P
            for j in range(t + 1):
                Pj = np.eye(7)
                for s_ in range(j + 1, t + 1):
                    Pj = Pj @ A[s_]
                St = St + b[j] * np.outer(v[j], kh[j]) @ Pj
            np.testing.assert_allclose(o[0, t, h], St @ qh[t], rtol=0, atol=1e-13)
            if t == 15:
                np.testing.assert_allclose(s[0, 0, h], St, rtol=0, atol=1e-13)


def test_linear_in_state_and_values():
    """For fixed q, k and gates, (state_in, v) -> (out, state_out) is linear."""
    x = _rand_problem(7, T=25)
    y = _rand_problem(8, T=25)
    c1, c2 = 0.75, -1.5
    args = (x["q"], x["k"])
    g = (x["log_alpha"], x["beta"])
    o1, s1 = oracle.forward(*args, x["v"], *g, x["state_in"], "fwd")
    o2, s2 = oracle.forward(*args, y["v"], *g, y["state_in"], "fwd")
    vm = (c1 * x["v"].astype(np.float64) + c2 * y["v"].astype(np.float64)).astype(np.float32)
    sm = (c1 * x["state_in"].astype(np.float64) + c2 * y["state_in"].astype(np.float64)).astype(np.float32)
    # c1, c2 are exact binary fractions, but fp32 inputs of the combination are rounded:
    # compare against the combination of the outputs with the rounded inputs' tolerance
    o3, s3 = oracle.forward(*args, vm, *g, sm, "fwd")
    np.testing.assert_allclose(o3, c1 * o1 + c2 * o2, rtol=0, atol=2e-6)
    np.testing.assert_allclose(s3, c1 * s1 + c2 * s2, rtol=0, atol=2e-6)
    # exact version: scaling by a power of two is exact in fp32
    o4, s4 = oracle.forward(*args, x["v"] * 4, *g, x["state_in"] * 4, "fwd")
    np.testing.assert_allclose(o4, 4 * o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(s4, 4 * s1, rtol=0, atol=1e-14)


def test_reverse_is_flipped_forward_and_bidirectional_is_sum():
    x = _rand_problem(9, T=29, direction="bi")
    q, k, v, la, bt, s0 = x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"]
    o_r, s_r = oracle.forward(q, k, v, la[1:], bt[1:], s0[1:], "rev")
    f = lambda a, ax: np.ascontiguousarray(np.flip(a, axis=ax))
    o_f, s_f = oracle.forward(f(q, 1), f(k, 1), f(v, 1), f(la[1:], 2), f(bt[1:], 2), s0[1:], "fwd")
    np.testing.assert_allclose(o_r, f(o_f, 1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(s_r, s_f, rtol=0, atol=1e-15)
    o_fw, s_fw = oracle.forward(q, k, v, la[:1], bt[:1], s0[:1], "fwd")
    o_b, s_b = oracle.forward(q, k, v, la, bt, s0, "bi")
    np.testing.assert_allclose(o_b, o_fw + o_r, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(s_b[0], s_fw[0])
    np.testing.assert_array_equal(s_b[1], s_r[0])


def test_streaming_split_equals_one_call():
    """State carried frame to frame equals one call over the concatenation."""
    x = _rand_problem(10, T=50, H=3)
    o, s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd")
    st = x["state_in"].astype(np.float64)
    outs = []
    for a, b in ((0, 13), (13, 14), (14, 50)):
        sl = slice(a, b)
        # the oracle takes a float32 state: carry in double through a float64 path
        o_i, st_new = oracle.forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["log_alpha"][:, :, sl],
                                     x["beta"][:, :, sl], st.astype(np.float32), "fwd")
        outs.append(o_i)
        st = st_new
    # the carried state is rounded to fp32 between calls, so allow fp32-level error
    np.testing.assert_allclose(np.concatenate(outs, axis=1), o, rtol=0, atol=1e-6)
    np.testing.assert_allclose(st, s, rtol=0, atol=1e-6)
    # exact version with zero state and split where the state is exactly representable:
    # a = 0 at the split token resets the state, so frames are independent
    la = x["log_alpha"].copy()
    la[:, :, 20] = -1e3
    o_full, _ = oracle.forward(x["q"], x["k"], x["v"], la, x["beta"], None, "fwd")
    o_tail, _ = oracle.forward(x["q"][:, 20:], x["k"][:, 20:], x["v"][:, 20:], la[:, :, 20:],
                               x["beta"][:, :, 20:], None, "fwd")
    np.testing.assert_array_equal(o_full[:, 20:], o_tail)


def test_zero_decay_closed_form():
    """a = 0 (log_alpha = -1e3): o_t = beta_t (q^_t . k^_t) v_t and S_T = beta v k^^T."""
    x = _rand_problem(11, T=21)
    la = np.full_like(x["log_alpha"], -1e3)
    o, s = oracle.forward(x["q"], x["k"], x["v"], la, x["beta"], x["state_in"], "fwd")
    qh, kh = _unit(x["q"][0].astype(np.float64)), _unit(x["k"][0].astype(np.float64))
    b = x["beta"][0, 0].astype(np.float64)
    ref = (b * np.sum(qh * kh, -1))[..., None] * x["v"][0]
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-15)
    for h in range(2):
        np.testing.assert_allclose(s[0, 0, h], b[-1, h] * np.outer(x["v"][0, -1, h], kh[-1, h]), atol=1e-15)


def test_zero_key_token_only_decays():
    """A zero key has no direction: k^ = 0, the step only decays the state."""
    x = _rand_problem(12, T=3)
    k = x["k"].copy()
    k[:, 1] = 0
    o, s = oracle.forward(x["q"][:, 1:2], k[:, 1:2], x["v"][:, 1:2], x["log_alpha"][:, :, 1:2],
                          x["beta"][:, :, 1:2], x["state_in"], "fwd")
    a = np.exp(x["log_alpha"][0, 0, 1].astype(np.float64))
    np.testing.assert_allclose(s[0, 0], a[:, None, None] * x["state_in"][0, 0], rtol=1e-15, atol=0)


def test_empty_sequence_passes_state_through():
    x = _rand_problem(13, T=4)
    sl = slice(0, 0)
    o, s = oracle.forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["log_alpha"][:, :, sl],
                          x["beta"][:, :, sl], x["state_in"], "fwd")
    assert o.shape == (1, 0, 2, 6)
    np.testing.assert_array_equal(s, x["state_in"].astype(np.float64))


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("la_shift", [3.0, -5.0])
def test_chunked_form_matches_token_oracle(direction, la_shift):
    """The independent chunked rewriting agrees to ~1e-12 for every chunk size, with tails."""
    x = _rand_problem(14, T=203, dk=16, dv=12, direction=direction, la_shift=la_shift)
    o, s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction)
    scale = np.sqrt(np.mean(o ** 2))
    for C in (16, 32, 64, 128):
        o2, s2 = chunked_ref.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"],
                                     direction, C)
        assert np.abs(o2 - o).max() <= 1e-12 * max(scale, 1)
        assert np.abs(s2 - s).max() <= 1e-12 * max(np.abs(s).max(), 1)


def test_bf16_inputs_are_widened_exactly():
    w = synth.WORKLOADS["tiny"].replace(dtype="bf16", T=40)
    x = synth.generate(w)
    o1, s1 = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None, "fwd")
    qf, kf, vf = (synth.bf16_to_f32(x[n]) for n in "qkv")
    o2, s2 = oracle.forward(qf, kf, vf, x["log_alpha"], x["beta"], None, "fwd")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_forward_heads_matches_full_run():
    x = _rand_problem(15, B=2, H=3, T=20, direction="bi")
    o, s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi")
    heads = [(1, 2), (0, 1)]
    oh, sh = oracle.forward_heads(x, heads, "bi")
    for i, (b, h) in enumerate(heads):
        np.testing.assert_array_equal(oh[i], o[b, :, h])
        np.testing.assert_array_equal(sh[:, i], s[:, b, h])


def _bidirectional_linear_attention(q, k, v, la_f, bt_f, la_r, bt_r, incl_f, incl_r):
    """Brute-force bidirectional gated linear attention (no erase), one chain.

    Every pair (t, s) written out with its explicit product of gates: the
    forward scan brings token s <= t (s < t when exclusive) with weight
    prod_{r=s+1..t} a_r, the reverse scan token s >= t (s > t when exclusive)
    with weight prod_{r=t..s-1} a'_r.
    """
    qh, kh = _unit(q.astype(np.float64)), _unit(k.astype(np.float64))
    af, ar = np.exp(la_f.astype(np.float64)), np.exp(la_r.astype(np.float64))
    T = q.shape[0]
    out = np.zeros((T, v.shape[1]))
    for t in range(T):
        for s in range(T):
            c = qh[t] @ kh[s]
            if s < t or (s == t and incl_f):
                out[t] += np.prod(af[s + 1:t + 1]) * bt_f[s] * c * v[s]
            if s > t or (s == t and incl_r):
                w = np.prod(ar[t:s]) if s > t else 1.0
                out[t] += w * bt_r[s] * c * v[s]
    return out


@pytest.mark.parametrize("exclusive", ["none", "fwd", "rev", "both"])
def test_exclusive_readout_erase_free_brute_force(exclusive):
    """Erase-free bidirectional scan with either readout against the pairwise sum.

    With only the reverse direction exclusive the two regions s <= t and s > t
    hold every token once; with both exclusive the token itself is in neither.
    """
    x = _rand_problem(21, T=27, direction="bi", state_std=0.0)
    o, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], None, "bi", erase=False,
                          exclusive=exclusive)
    incl_f = exclusive in ("none", "rev")
    incl_r = exclusive in ("none", "fwd")
    for h in range(2):
        ref = _bidirectional_linear_attention(
            x["q"][0, :, h], x["k"][0, :, h], x["v"][0, :, h],
            x["log_alpha"][0, 0, :, h], x["beta"][0, 0, :, h].astype(np.float64),
            x["log_alpha"][1, 0, :, h], x["beta"][1, 0, :, h].astype(np.float64), incl_f, incl_r)
        np.testing.assert_allclose(o[0, :, h], ref, rtol=0, atol=1e-12)


def test_exclusive_partition_without_gates_is_noncausal_linear_attention():
    """a = 1, beta = 1, reverse exclusive: out = (Q^ K^^T) V over the whole sequence."""
    x = _rand_problem(22, T=31, direction="bi", state_std=0.0)
    la, bt = np.zeros_like(x["log_alpha"]), np.ones_like(x["beta"])
    o, _ = oracle.forward(x["q"], x["k"], x["v"], la, bt, None, "bi", erase=False, exclusive="rev")
    qh, kh = _unit(x["q"][0].astype(np.float64)), _unit(x["k"][0].astype(np.float64))
    ref = np.einsum("thk,shk,shv->thv", qh, kh, x["v"][0].astype(np.float64))
    np.testing.assert_allclose(o[0], ref, rtol=0, atol=1e-12)


def test_exclusive_readout_ignores_the_tokens_own_write():
    """Changing token t's key, value and write strength leaves exclusive readouts at t untouched."""
    x = _rand_problem(23, T=19, direction="bi")
    t = 7
    y = {n: a.copy() for n, a in x.items()}
    y["k"][:, t] = -2.0 * y["k"][:, t] + 0.5
    y["v"][:, t] += 3.0
    y["beta"][:, :, t] = 1.0 - y["beta"][:, :, t]
    args = lambda d, sl: (d["q"], d["k"], d["v"], d["log_alpha"][sl], d["beta"][sl], d["state_in"][sl])
    # both exclusive: the two regions exclude t, bit for bit
    o1, _ = oracle.forward(*args(x, slice(None)), "bi", exclusive="both")
    o2, _ = oracle.forward(*args(y, slice(None)), "bi", exclusive="both")
    np.testing.assert_array_equal(o1[:, t], o2[:, t])
    assert np.abs(o1[:, t + 1] - o2[:, t + 1]).max() > 1e-3
    # forward exclusive: every readout up to t; reverse exclusive: from t on
    o1, _ = oracle.forward(*args(x, slice(0, 1)), "fwd", exclusive="fwd")
    o2, _ = oracle.forward(*args(y, slice(0, 1)), "fwd", exclusive="fwd")
    np.testing.assert_array_equal(o1[:, :t + 1], o2[:, :t + 1])
    o1, _ = oracle.forward(*args(x, slice(1, 2)), "rev", exclusive="rev")
    o2, _ = oracle.forward(*args(y, slice(1, 2)), "rev", exclusive="rev")
    np.testing.assert_array_equal(o1[:, t:], o2[:, t:])
    # the inclusive readout does see the token
    o1, _ = oracle.forward(*args(x, slice(0, 1)), "fwd")
    o2, _ = oracle.forward(*args(y, slice(0, 1)), "fwd")
    assert np.abs(o1[:, t] - o2[:, t]).max() > 1e-3
    # the exclusive option changes readouts only: final states are the inclusive ones
    _, s1 = oracle.forward(*args(x, slice(None)), "bi")
    _, s2 = oracle.forward(*args(x, slice(None)), "bi", exclusive="both")
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("t", [0, 1, 12, 24])
def test_exclusive_readout_is_decayed_prefix_state(t):
    """Delta rule: exclusive o_t = a_t S_{t-1} q^_t with S_{t-1} the state after tokens < t.

    S_{t-1} comes from a separate call over the prefix (its final state); the
    reverse direction mirrors this with the suffix after t.
    """
    x = _rand_problem(24, T=25, direction="bi")
    q, k, v, la, bt, s0 = x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"]
    T = q.shape[1]
    qh = _unit(q[0, t].astype(np.float64))
    of, _ = oracle.forward(q, k, v, la[:1], bt[:1], s0[:1], "fwd", exclusive="fwd")
    _, sp = oracle.forward(q[:, :t], k[:, :t], v[:, :t], la[:1, :, :t], bt[:1, :, :t], s0[:1], "fwd")
    a = np.exp(la[0, 0, t].astype(np.float64))
    ref = a[:, None] * np.einsum("hvk,hk->hv", sp[0, 0], qh)
    np.testing.assert_allclose(of[0, t], ref, rtol=0, atol=1e-13)
    orv, _ = oracle.forward(q, k, v, la[1:], bt[1:], s0[1:], "rev", exclusive="rev")
    _, ss = oracle.forward(q[:, t + 1:], k[:, t + 1:], v[:, t + 1:], la[1:, :, t + 1:], bt[1:, :, t + 1:],
                           s0[1:], "rev")
    a = np.exp(la[1, 0, t].astype(np.float64))
    ref = a[:, None] * np.einsum("hvk,hk->hv", ss[0, 0], qh)
    np.testing.assert_allclose(orv[0, t], ref, rtol=0, atol=1e-13)
    assert T == 25


def test_exclusive_text_state_enters_once():
    """Text folded in as S_T/2 per direction, nothing written, no decay: out = S_T q^_t.

    A single token reads a_0 S_in q^_0 from each direction whatever its write.
    """
    x = _rand_problem(25, T=9, direction="bi")
    S_T = np.random.default_rng(5).standard_normal((1, 2, 6, 8)).astype(np.float32)
    half = np.stack([S_T / 2, S_T / 2])
    la, bt = np.zeros_like(x["log_alpha"]), np.zeros_like(x["beta"])
    o, _ = oracle.forward(x["q"], x["k"], x["v"], la, bt, half, "bi", exclusive="both")
    qh = _unit(x["q"][0].astype(np.float64))
    np.testing.assert_allclose(o[0], np.einsum("hvk,thk->thv", S_T[0].astype(np.float64), qh), rtol=0,
                               atol=1e-13)
    sl = slice(3, 4)
    o, _ = oracle.forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["log_alpha"][:, :, sl],
                          x["beta"][:, :, sl], x["state_in"], "bi", exclusive="both")
    a = np.exp(x["log_alpha"][:, 0, 3].astype(np.float64))  # [dirs, H]
    S = x["state_in"][:, 0].astype(np.float64)                 # [dirs, H, dv, dk]
    ref = np.einsum("dh,dhvk,hk->hv", a, S, qh[3])
    np.testing.assert_allclose(o[0, 0], ref, rtol=0, atol=1e-13)


def test_reset_gate_makes_windows_independent():
    """log_alpha = -1000 gives a = 0 exactly, so a direction's memory restarts at that
    token: with a forward reset at a window's first token and a reverse reset at its
    last, the bidirectional outputs of the window equal a run on the window alone
    (the method the longest-sequence GPU test relies on)."""
    x = _rand_problem(26, T=400, H=2, dk=16, dv=12, direction="bi")
    la = x["log_alpha"].copy()
    W, m, T = 40, 181, 400
    la[1, :, W - 1] = -1000.0
    la[0, :, m] = -1000.0
    la[1, :, m + W - 1] = -1000.0
    la[0, :, T - W] = -1000.0
    q, k, v, bt, s0 = x["q"], x["k"], x["v"], x["beta"], x["state_in"]
    o, s = oracle.forward(q, k, v, la, bt, s0, "bi")
    zero = np.zeros_like(s0[:1])
    for t0, t1, st in ((0, W, np.concatenate([s0[:1], zero])), (m, m + W, None),
                       (T - W, T, np.concatenate([zero, s0[1:]]))):
        sl = slice(t0, t1)
        ow, sw = oracle.forward(q[:, sl], k[:, sl], v[:, sl], la[:, :, sl], bt[:, :, sl], st, "bi")
        np.testing.assert_allclose(o[:, sl], ow, rtol=0, atol=1e-13)
        if t0 == 0:
            np.testing.assert_allclose(s[1], sw[1], rtol=0, atol=1e-13)
        if t1 == T:
            np.testing.assert_allclose(s[0], sw[0], rtol=0, atol=1e-13)
    # without the resets the windows do depend on the rest
    o2, _ = oracle.forward(q, k, v, x["log_alpha"], bt, s0, "bi")
    ow, _ = oracle.forward(q[:, m:m + W], k[:, m:m + W], v[:, m:m + W], x["log_alpha"][:, :, m:m + W],
                           bt[:, :, m:m + W], None, "bi")
    assert np.abs(o2[:, m:m + W] - ow).max() > 1e-6


def test_hand_worked_example_exclusive_readouts():
    """The two-token example's exclusive readouts, worked by hand
    (tests/golden/hand_worked_2token.json, "derivation_exclusive")."""
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_2token.json")))
    inp, exp = g["inputs"], g["expected_exclusive"]
    q = np.array(inp["q"], np.float32)[None, :, None, :]
    k = np.array(inp["k"], np.float32)[None, :, None, :]
    v = np.array(inp["v"], np.float32)[None, :, None, :]
    la = np.log(np.array([inp["alpha_fwd"], inp["alpha_rev"]], np.float64)).astype(np.float32)[:, None, :, None]
    bt = np.array([inp["beta_fwd"], inp["beta_rev"]], np.float32)[:, None, :, None]
    tol = dict(rtol=0, atol=1e-7)
    o, _ = oracle.forward(q, k, v, la[:1], bt[:1], None, "fwd", exclusive="fwd")
    np.testing.assert_allclose(o[0, :, 0], exp["out_fwd"], **tol)
    o, _ = oracle.forward(q, k, v, la[1:], bt[1:], None, "rev", exclusive="rev")
    np.testing.assert_allclose(o[0, :, 0], exp["out_rev"], **tol)
    for mode, key in (("both", "out_bi_both"), ("rev", "out_bi_rev"), ("fwd", "out_bi_fwd")):
        o, _ = oracle.forward(q, k, v, la, bt, None, "bi", exclusive=mode)
        np.testing.assert_allclose(o[0, :, 0], exp[key], **tol)


def test_readout_epilogue_hand_worked():
    """The token scan's readout epilogue, worked by hand on rows where
    mean(o^2) and eps are comparable: o = (1.5e-3, 2e-3) has mean(o^2) =
    3.125e-6; with eps = 3.125e-6, sqrt(mean + eps) = 2.5e-3, so an open
    gate (z = 60) and unit weights give (0.6, 0.8), a gate at z = 0 halves
    it, weights (2, -1) give (1.2, -0.8), and z = ln 3 multiplies by 3/4.
    A row of zeros stays zero (eps > 0); eps elsewhere (sqrt(mean) + eps, or
    none) is far from these values.  Two rows of one head are normalised
    separately (the mean runs over one row's channels only)."""
    o = np.array([[1.5e-3, 2e-3], [3.0, 4.0]])
    eps = 3.125e-6
    g_open = np.full((2, 2), 60.0, np.float32)
    y = oracle.readout_epilogue(o, g_open, [1.0, 1.0], eps)
    np.testing.assert_allclose(y[0], [0.6, 0.8], rtol=1e-12, atol=0)
    # second row: mean(o^2) = 12.5, eps negligible: o / sqrt(12.5)
    np.testing.assert_allclose(y[1], np.array([3.0, 4.0]) / np.sqrt(12.5 + eps), rtol=1e-12)
    np.testing.assert_allclose(oracle.readout_epilogue(o[:1], np.zeros((1, 2), np.float32), [1.0, 1.0], eps)[0],
                               [0.3, 0.4], rtol=1e-12)
    np.testing.assert_allclose(oracle.readout_epilogue(o[:1], g_open[:1], [2.0, -1.0], eps)[0], [1.2, -0.8],
                               rtol=1e-12)
    z3 = np.full((1, 2), np.log(3.0), np.float32)  # sigmoid(ln 3) = 3/4 up to the float32 rounding of ln 3
    np.testing.assert_allclose(oracle.readout_epilogue(o[:1], z3, [1.0, 1.0], eps)[0], [0.45, 0.6], rtol=1e-7)
    assert np.all(oracle.readout_epilogue(np.zeros((1, 2)), g_open[:1], [1.0, 1.0], eps) == 0)
    for alt in (o[0] / (np.sqrt(np.mean(o[0] ** 2)) + eps), o[0] / np.sqrt(np.mean(o[0] ** 2))):
        assert np.max(np.abs(alt - [0.6, 0.8])) > 0.2
    # bf16 gate bit patterns are widened exactly: 0x3F80 is 1.0
    yb = oracle.readout_epilogue(o[:1], np.full((1, 2), 0x3F80, np.uint16), [1.0, 1.0], eps)[0]
    np.testing.assert_allclose(yb, np.array([0.6, 0.8]) / (1.0 + np.exp(-1.0)), rtol=1e-12)
