"""Pins of the frame-wise delta operator's oracle (oracle/vda.py), CPU only.

Each pin checks the oracle against something other than its own formula:
  * one token per frame: the closed form reduces (Sherman-Morrison) to the
    token delta rule with write strength beta / (1 + beta) -- checked against
    the independent C token oracle;
  * least squares: every frame's state has a zero gradient of the objective
    the page states ("Video DeltaNet", "Methodology in Plain English": stay
    close to the decayed memory while fitting the frame's associations);
  * hand-worked frames: orthonormal keys give a diagonal inverse, and two
    identical keys average their values with the decayed memory;
  * order of the tokens inside a frame does not matter;
  * non-expansiveness ("Key Contributions" item 2) even where the additive
    per-token update I - A_t expands ("Main Findings": eigenvalues leave
    [-1, 1] once lambda_max(A_t) > 2);
  * beta = 0 is pure decay; reverse is flip-forward-flip; bidirectional is the
    sum of the two scans.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import vda


def _inputs(T=90, frame=30, H=2, d=16, direction="fwd", shift=-3.0, std=0.1, seed=1):
    w = synth.Workload("vda", 1, H, T, d, d, "f32", direction, shift, std, seed)
    return synth.generate_frames(w, frame)


def test_one_token_frames_equal_the_token_delta_rule():
    for direction in ("fwd", "rev", "bi"):
        x = _inputs(T=40, frame=1, direction=direction)
        o_vda, s_vda = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction, 1)
        b = x["beta"].astype(np.float64)
        b2 = (b / (1.0 + b)).astype(np.float32)
        # per-token gates: a frame of one token has its token's decay
        o_tok, s_tok = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], b2, x["state_in"], direction)
        # the transformed beta is rounded to fp32 for the C oracle: agreement to that precision
        assert np.max(np.abs(o_vda - o_tok)) <= 1e-6 * max(1.0, np.max(np.abs(o_tok)))
        assert np.max(np.abs(s_vda - s_tok)) <= 1e-6 * max(1.0, np.max(np.abs(s_tok)))


def test_every_frame_state_minimises_the_objective():
    x = _inputs(T=100, frame=32, direction="fwd")
    _, _, states = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd", 32,
                               return_states=True)
    q, k, v = (oracle.as_f32(x[n]).astype(np.float64) for n in ("q", "k", "v"))
    kh = k / np.maximum(np.linalg.norm(k, axis=-1, keepdims=True), 1e-6)
    for h in range(2):
        S_prev = x["state_in"][0, 0, h].astype(np.float64)
        for f in range(states.shape[3]):
            t0, t1 = 32 * f, min(100, 32 * (f + 1))
            a = np.exp(float(x["log_alpha"][0, 0, f, h]))
            S = states[0, 0, h, f]
            grad = S - a * S_prev
            for i in range(t0, t1):
                r = S @ kh[0, i, h] - v[0, i, h]
                grad += float(x["beta"][0, 0, i, h]) * np.outer(r, kh[0, i, h])
            assert np.max(np.abs(grad)) < 1e-10 * max(1.0, np.max(np.abs(S)))
            S_prev = S


def test_hand_worked_frames():
    # dk = dv = 2, one frame of two tokens, a = 0.5, S_in = [[1, 2], [3, 4]]
    S0 = np.array([[1.0, 2.0], [3.0, 4.0]])
    v1, v2 = np.array([1.0, -1.0]), np.array([2.0, 0.5])
    # orthonormal keys e1, e2 with beta 1 and 3: column j becomes (a S0[:, j] + beta_j v_j) / (1 + beta_j)
    S = vda.frame_update(S0, 0.5, np.array([[1.0, 0.0], [0.0, 1.0]]), np.stack([v1, v2]), np.array([1.0, 3.0]))
    want = np.stack([(0.5 * S0[:, 0] + v1) / 2.0, (0.5 * S0[:, 1] + 3.0 * v2) / 4.0], axis=1)
    assert np.allclose(S, want, rtol=0, atol=1e-14)
    # two identical keys e1 with beta 1: the fitted column is the mean of a S0[:, 0], v1 and v2;
    # the orthogonal column keeps the decayed memory
    S = vda.frame_update(S0, 0.5, np.array([[1.0, 0.0], [1.0, 0.0]]), np.stack([v1, v2]), np.array([1.0, 1.0]))
    want = np.stack([(0.5 * S0[:, 0] + v1 + v2) / 3.0, 0.5 * S0[:, 1]], axis=1)
    assert np.allclose(S, want, rtol=0, atol=1e-14)


def test_token_order_inside_a_frame_does_not_matter():
    x = _inputs(T=64, frame=32, direction="bi", seed=3)
    o1, s1 = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 32)
    perm = np.concatenate([np.random.default_rng(0).permutation(32), 32 + np.random.default_rng(1).permutation(32)])
    y = dict(x)
    for n in ("q", "k", "v"):
        y[n] = x[n][:, perm]
    y["beta"] = x["beta"][:, :, perm]
    o2, s2 = vda.forward(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"], y["state_in"], "bi", 32)
    assert np.allclose(s1, s2, rtol=0, atol=1e-12)
    assert np.allclose(o1[:, perm], o2, rtol=0, atol=1e-12)


def test_transition_is_non_expansive_where_additive_writes_expand():
    rng = np.random.default_rng(5)
    d, n = 8, 40
    # keys bunched around one direction, beta = 1: lambda_max(A) well above 2
    base = rng.standard_normal(d)
    kh = base[None, :] + 0.2 * rng.standard_normal((n, d))
    kh /= np.linalg.norm(kh, axis=1, keepdims=True)
    A = kh.T @ kh
    assert np.max(np.linalg.eigvalsh(A)) > 2.0
    assert np.max(np.abs(np.linalg.eigvalsh(np.eye(d) - A))) > 1.0  # the additive form expands
    # the operator's transition (v = 0): S -> a S (I + A)^{-1}, never larger in spectral norm
    S = rng.standard_normal((d, d))
    for a in (1.0, 0.7):
        S1 = vda.frame_update(S, a, kh, np.zeros((n, d)), np.ones(n))
        assert np.linalg.norm(S1, 2) <= a * np.linalg.norm(S, 2) + 1e-12


def test_zero_beta_is_pure_decay():
    x = _inputs(T=60, frame=20, direction="fwd", seed=4)
    x["beta"] = np.zeros_like(x["beta"])
    o, s = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd", 20)
    a_tot = np.exp(np.sum(x["log_alpha"][0, 0].astype(np.float64), axis=0))  # [H]
    assert np.allclose(s[0, 0], x["state_in"][0, 0] * a_tot[:, None, None], rtol=1e-12, atol=0)
    q = oracle.as_f32(x["q"]).astype(np.float64)
    qh = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6)
    a_first = np.exp(x["log_alpha"][0, 0, 0].astype(np.float64))
    for h in range(2):
        want = qh[0, :20, h] @ (a_first[h] * x["state_in"][0, 0, h].astype(np.float64)).T
        assert np.allclose(o[0, :20, h], want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("T,frame", [(90, 30), (64, 16)])
def test_reverse_and_bidirectional(T, frame):
    x = _inputs(T=T, frame=frame, direction="bi", seed=6)
    o_bi, s_bi = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", frame)
    sl = lambda a, i: a[i:i + 1]
    o_f, s_f = vda.forward(x["q"], x["k"], x["v"], sl(x["log_alpha"], 0), sl(x["beta"], 0), sl(x["state_in"], 0),
                           "fwd", frame)
    o_r, s_r = vda.forward(x["q"], x["k"], x["v"], sl(x["log_alpha"], 1), sl(x["beta"], 1), sl(x["state_in"], 1),
                           "rev", frame)
    assert np.allclose(o_bi, o_f + o_r, rtol=0, atol=1e-12)
    assert np.allclose(s_bi[0], s_f[0]) and np.allclose(s_bi[1], s_r[0])
    # reverse = flip . forward . flip (T a multiple of the frame: frames map onto frames)
    fl = lambda a, ax: np.ascontiguousarray(np.flip(a, axis=ax))
    o_ff, s_ff = vda.forward(fl(x["q"], 1), fl(x["k"], 1), fl(x["v"], 1), fl(sl(x["log_alpha"], 1), 2),
                             fl(sl(x["beta"], 1), 2), sl(x["state_in"], 1), "fwd", frame)
    assert np.allclose(fl(o_ff, 1), o_r, rtol=0, atol=1e-12)
    assert np.allclose(s_ff, s_r, rtol=0, atol=1e-12)


# ---- additive frame writes (summed per-token corrections, keys / sqrt(U)) ----

def test_additive_one_token_frames_equal_the_token_delta_rule():
    # U = 1: the correction of the only token is the delta rule itself
    for direction in ("fwd", "rev", "bi"):
        x = _inputs(T=40, frame=1, direction=direction, seed=7)
        o1, s1 = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction, 1,
                             write="additive")
        o2, s2 = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction)
        assert np.max(np.abs(o1 - o2)) <= 1e-9 * max(1.0, np.max(np.abs(o2)))
        assert np.max(np.abs(s1 - s2)) <= 1e-9 * max(1.0, np.max(np.abs(s2)))


def test_additive_token_order_inside_a_frame_does_not_matter():
    x = _inputs(T=64, frame=32, direction="bi", seed=8)
    o1, s1 = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 32, write="additive")
    perm = np.concatenate([np.random.default_rng(2).permutation(32), 32 + np.random.default_rng(3).permutation(32)])
    y = dict(x)
    for n in ("q", "k", "v"):
        y[n] = x[n][:, perm]
    y["beta"] = x["beta"][:, :, perm]
    o2, s2 = vda.forward(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"], y["state_in"], "bi", 32, write="additive")
    assert np.allclose(s1, s2, rtol=0, atol=1e-12)
    assert np.allclose(o1[:, perm], o2, rtol=0, atol=1e-12)


def test_additive_scaled_write_is_non_expansive_where_the_unscaled_one_expands():
    rng = np.random.default_rng(9)
    d, n = 8, 40
    kh = rng.standard_normal(d)[None, :] + 0.2 * rng.standard_normal((n, d))
    kh /= np.linalg.norm(kh, axis=1, keepdims=True)
    S = rng.standard_normal((d, d))
    # unscaled: S (I - A) with lambda_max(A) > 2 grows along the top eigenvector
    A = kh.T @ kh
    top = np.linalg.eigh(A)[1][:, -1]
    S_top = np.outer(rng.standard_normal(d), top)
    assert np.linalg.norm(S_top @ (np.eye(d) - A), 2) > np.linalg.norm(S_top, 2)
    # scaled by 1/sqrt(U): never larger, for any beta in [0, 1]
    for beta in (np.ones(n), rng.uniform(0, 1, n)):
        for a in (1.0, 0.8):
            S1 = vda.frame_update_additive(S, a, kh, np.zeros((n, d)), beta)
            assert np.linalg.norm(S1, 2) <= a * np.linalg.norm(S, 2) + 1e-12
            S2 = vda.frame_update_additive(S_top, a, kh, np.zeros((n, d)), beta)
            assert np.linalg.norm(S2, 2) <= a * np.linalg.norm(S_top, 2) + 1e-12


# ---- disjoint-region readout (lag) ----

@pytest.mark.parametrize("lag", [1, 2])
def test_lag_on_one_token_frames_is_the_lagged_token_readout(lag):
    # forward, frames of one token: o_t = S_{t-lag} q^_t, where S_j is the token
    # delta rule's state after token j (beta / (1 + beta)), taken from the C
    # oracle run on the prefix; the initial state for t < lag
    x = _inputs(T=12, frame=1, direction="fwd", seed=10)
    o, _ = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd", 1, lag=lag)
    b2 = (x["beta"].astype(np.float64) / (1.0 + x["beta"].astype(np.float64))).astype(np.float32)
    q = oracle.as_f32(x["q"]).astype(np.float64)
    qh = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6)
    for t in range(12):
        j = t - lag + 1  # tokens 0 .. t-lag written
        if j <= 0:
            S = x["state_in"][0, 0].astype(np.float64)
        else:
            _, s = oracle.forward(x["q"][:, :j], x["k"][:, :j], x["v"][:, :j], x["log_alpha"][:, :, :j], b2[:, :, :j],
                                  x["state_in"], "fwd")
            S = s[0, 0]
        want = np.einsum("hvk,hk->hv", S, qh[0, t])
        assert np.allclose(o[0, t], want, rtol=0, atol=2e-6 * max(1.0, np.max(np.abs(want))))


@pytest.mark.parametrize("lag", [0, 1, 3])
def test_text_state_enters_once(lag):
    # no writes (beta = 0) and no decay: every token reads S_T/2 from each direction
    x = _inputs(T=48, frame=8, direction="bi", seed=11)
    x["beta"] = np.zeros_like(x["beta"])
    x["log_alpha"] = np.zeros_like(x["log_alpha"])
    S_T = np.random.default_rng(4).standard_normal((1, 2, 16, 16))
    half = np.stack([S_T / 2, S_T / 2])
    o, _ = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], half, "bi", 8, lag=lag)
    q = oracle.as_f32(x["q"]).astype(np.float64)
    qh = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6)
    assert np.allclose(o, np.einsum("bhvk,bthk->bthv", S_T, qh), rtol=0, atol=1e-12)


def test_lagged_readouts_cover_disjoint_regions():
    # lag 2, frames of 8 tokens, 6 frames: frame 2's writes reach the forward
    # readout of frames >= 4 and the reverse readout of frames <= 0 only
    x = _inputs(T=48, frame=8, direction="bi", seed=12)
    o1, _ = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 8, lag=2)
    y = {n: np.array(x[n], copy=True) for n in ("k", "v", "beta")}
    rng = np.random.default_rng(5)
    y["k"][:, 16:24] = rng.standard_normal(y["k"][:, 16:24].shape).astype(np.float32)
    y["v"][:, 16:24] = rng.standard_normal(y["v"][:, 16:24].shape).astype(np.float32)
    y["beta"][:, :, 16:24] = rng.uniform(0, 1, y["beta"][:, :, 16:24].shape).astype(np.float32)
    o2, _ = vda.forward(x["q"], y["k"], y["v"], x["log_alpha"], y["beta"], x["state_in"], "bi", 8, lag=2)
    same = np.all(np.isclose(o1, o2, rtol=0, atol=1e-13), axis=(0, 2, 3)).reshape(6, 8).all(axis=1)
    assert list(same) == [False, True, True, True, False, False]


def test_lag_past_every_frame_reads_the_initial_states():
    x = _inputs(T=40, frame=8, direction="bi", seed=13)
    o, _ = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 8, lag=5)
    q = oracle.as_f32(x["q"]).astype(np.float64)
    qh = q / np.maximum(np.linalg.norm(q, axis=-1, keepdims=True), 1e-6)
    S = x["state_in"].astype(np.float64).sum(axis=0)
    assert np.allclose(o, np.einsum("bhvk,bthk->bthv", S, qh), rtol=0, atol=1e-12)


# ---- readout epilogue (RMS normalisation and sigmoid gate) ----

def _epilogue_case(seed=14):
    x = _inputs(T=40, frame=8, direction="bi", seed=seed)
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((1, 40, 2, 16)).astype(np.float32)
    wgt = rng.uniform(0.5, 1.5, 16)
    return x, z, wgt


def test_epilogue_is_invariant_to_the_scale_of_the_readout():
    x, z, wgt = _epilogue_case()
    o1, _ = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 8, gate=z,
                        norm_weight=wgt, norm_eps=0.0)
    y = dict(x)
    y["v"] = (x["v"] * 4.0).astype(np.float32)
    y["state_in"] = (x["state_in"] * 4.0).astype(np.float32)
    o2, _ = vda.forward(y["q"], y["k"], y["v"], y["log_alpha"], y["beta"], y["state_in"], "bi", 8, gate=z,
                        norm_weight=wgt, norm_eps=0.0)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-14)


def test_epilogue_gives_unit_rms_per_token_and_head_with_an_open_gate():
    x, z, _ = _epilogue_case(15)
    o, _ = vda.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 8,
                       gate=np.full_like(z, 60.0), norm_weight=np.ones(16), norm_eps=0.0)
    assert np.allclose(np.sqrt(np.mean(o * o, axis=-1)), 1.0, rtol=0, atol=1e-12)


def test_epilogue_gate_and_weights():
    x, z, wgt = _epilogue_case(16)
    args = (x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 8)
    open_, _ = vda.forward(*args, gate=np.full_like(z, 60.0), norm_weight=np.ones(16), norm_eps=1e-6)
    half, _ = vda.forward(*args, gate=np.zeros_like(z), norm_weight=np.ones(16), norm_eps=1e-6)
    assert np.allclose(half, open_ / 2, rtol=1e-12, atol=0)  # sigmoid(0) = 1/2
    one_hot = np.zeros(16)
    one_hot[5] = 3.0
    sel, _ = vda.forward(*args, gate=np.full_like(z, 60.0), norm_weight=one_hot, norm_eps=1e-6)
    assert np.allclose(sel[..., 5], 3.0 * open_[..., 5], rtol=1e-12, atol=0)
    assert np.all(np.delete(sel, 5, axis=-1) == 0)


def test_epilogue_eps_sits_inside_the_root_hand_worked():
    """Where eps stands in the RMS normalisation, worked by hand at a size
    where mean(o^2) and eps are comparable.  One frame of one token, no
    initial state, beta = 1, k = q = e1 (dk = 2), v = (3e-3, 4e-3) (dv = 2):
    A = e1 e1^T, B = v e1^T, S = B (I + A)^-1 = (v / 2) e1^T, so o = S q^ =
    (1.5e-3, 2e-3) and mean(o^2) = (2.25e-6 + 4e-6) / 2 = 3.125e-6.  With
    eps = 3.125e-6, sqrt(mean + eps) = sqrt(6.25e-6) = 2.5e-3 and an open
    gate (z = 60: sigmoid = 1 in double) and unit weights, y = o / 2.5e-3 =
    (0.6, 0.8).  The other placements give other values: sqrt(mean) + eps
    -> (0.8470, 1.1294), no eps -> (0.8485, 1.1314).  Closed gate z = 0 halves
    it: (0.3, 0.4); weights (2, -1) give (1.2, -0.8)."""
    q = np.array([1.0, 0.0], np.float32).reshape(1, 1, 1, 2)
    k = q.copy()
    v = np.array([3e-3, 4e-3], np.float64).astype(np.float32).reshape(1, 1, 1, 2)
    la = np.zeros((1, 1, 1, 1), np.float32)
    bt = np.ones((1, 1, 1, 1), np.float32)
    vv = v.astype(np.float64).ravel()  # the float32 inputs as the oracle sees them
    o = vv / 2.0
    eps = float(np.mean(o * o))  # 3.125e-6 up to the float32 rounding of v
    assert abs(eps - 3.125e-6) < 1e-12
    def run(z, w):
        y, _ = vda.forward(q, k, v, la, bt, None, "fwd", 1, gate=np.full((1, 1, 1, 2), z, np.float32),
                           norm_weight=np.asarray(w, np.float64), norm_eps=eps)
        return y.ravel()
    want = o / np.sqrt(2.0 * eps)
    assert np.allclose(want, [0.6, 0.8], rtol=0, atol=2e-7)
    np.testing.assert_allclose(run(60.0, [1.0, 1.0]), want, rtol=1e-13, atol=0)
    np.testing.assert_allclose(run(0.0, [1.0, 1.0]), want / 2, rtol=1e-13, atol=0)
    np.testing.assert_allclose(run(60.0, [2.0, -1.0]), want * [2.0, -1.0], rtol=1e-13, atol=0)
    # the other placements are far from the oracle's values
    for alt in (o / (np.sqrt(eps) + eps), o / np.sqrt(eps)):
        assert np.max(np.abs(run(60.0, [1.0, 1.0]) - alt)) > 0.2


def test_reset_gate_makes_frame_windows_independent():
    """A per-frame log-gate of -1000 gives a = 0 exactly: S_t = B_t (I + A_t)^-1
    whatever came before.  With a forward reset at a window's first frame and a
    reverse reset at its last, the window's outputs equal a run on it alone
    (the method of the longest-sequence GPU test of the frame-wise operator)."""
    frame, n = 20, 3
    x = _inputs(T=215, frame=frame, direction="bi", shift=3.0)
    la = x["log_alpha"].copy()
    NF = la.shape[2]
    fm = 5
    la[1, :, n - 1] = -1000.0
    la[0, :, fm] = -1000.0
    la[1, :, fm + n - 1] = -1000.0
    la[0, :, NF - n] = -1000.0
    q, k, v, bt, s0 = x["q"], x["k"], x["v"], x["beta"], x["state_in"]
    T = q.shape[1]
    o, s = vda.forward(q, k, v, la, bt, s0, "bi", frame)
    zero = np.zeros_like(s0[:1])
    for f0, f1, st in ((0, n, np.concatenate([s0[:1], zero])), (fm, fm + n, None),
                       (NF - n, NF, np.concatenate([zero, s0[1:]]))):
        t0, t1 = f0 * frame, min(T, f1 * frame)
        sl = slice(t0, t1)
        ow, sw = vda.forward(q[:, sl], k[:, sl], v[:, sl], la[:, :, f0:f1], bt[:, :, sl], st, "bi", frame)
        np.testing.assert_allclose(o[:, sl], ow, rtol=0, atol=1e-12)
        if f0 == 0:
            np.testing.assert_allclose(s[1], sw[1], rtol=0, atol=1e-12)
        if f1 == NF:
            np.testing.assert_allclose(s[0], sw[0], rtol=0, atol=1e-12)
    # without the resets a window depends on the rest
    o2, _ = vda.forward(q, k, v, x["log_alpha"], bt, s0, "bi", frame)
    t0, t1 = fm * frame, (fm + n) * frame
    ow, _ = vda.forward(q[:, t0:t1], k[:, t0:t1], v[:, t0:t1], x["log_alpha"][:, :, fm:fm + n], bt[:, :, t0:t1],
                        None, "bi", frame)
    assert np.abs(o2[:, t0:t1] - ow).max() > 1e-6
