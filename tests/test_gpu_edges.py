"""GPU edge cases of the scan, each against the double-precision oracle at the
tolerances of tests/gdn_testutil.py (or exactly, where the result is exact):

* sequence lengths around the chunk size (one token, a partial chunk, one
  full chunk, one chunk plus one token) in every direction;
* an empty sequence (the state passes through unchanged);
* no initial state, and the state carried in place (state_out is state_in);
* degenerate gates: beta = 0 (pure decay, no writes), log_alpha = 0 (the
  ungated delta rule), log_alpha = -50 (the state is forgotten at every token);
* all-zero q and k rows (the norm clamp keeps them zero);
* bitwise repeatability of two identical calls.
"""
import numpy as np
import pytest

import oracle
import synth
from gdn_testutil import TOL, check, run_gpu, to_torch

pytestmark = pytest.mark.gpu


def _inputs(dtype, direction, T, B=1, H=2, d=64, state_std=0.05, seed=11):
    w = synth.Workload("edge", B, H, T, d, d, dtype, direction, 3.0, state_std, seed)
    return w, synth.generate(w)


def _compare(x, w, tol=None, **kw):
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], w.direction)
    out, s = run_gpu(x, w.direction, **kw)
    tol = tol or TOL[w.dtype]
    e1 = check(out, ref, tol, f"out {w}")
    e2 = check(s, ref_s, tol, f"state {w}")
    print(f"\n{w.dtype} {w.direction} T={w.T}: out {e1:.2e} state {e2:.2e}", flush=True)


@pytest.mark.parametrize("T", [1, 17, 64, 65, 128])
@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
def test_lengths_around_one_chunk(T, direction):
    w, x = _inputs("bf16", direction, T, d=128)
    _compare(x, w)


@pytest.mark.parametrize("T", [1, 31, 33])
def test_lengths_around_small_chunk_fp32(T):
    w, x = _inputs("f32", "bi", T)
    _compare(x, w, chunk=32)


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
def test_empty_sequence_passes_state_through(direction):
    import torch

    import gated_delta_rule_scan_amd as gdn

    dirs = 2 if direction == "bi" else 1
    rng = np.random.default_rng(3)
    s_in = rng.standard_normal((dirs, 1, 2, 64, 64)).astype(np.float32)
    empty = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((dirs, 1, 0, 2), dtype=torch.float32, device="cuda")
    out, s_out = gdn.forward(empty, empty, empty, g, g, to_torch(s_in), direction)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (1, 0, 2, 64)
    assert np.array_equal(s_out.cpu().numpy(), s_in)


def test_no_initial_state():
    w, x = _inputs("bf16", "bi", 150, d=128, state_std=0.0)
    assert x["state_in"] is None
    _compare(x, w)


def test_state_carried_in_place():
    """state_out may be the state_in buffer itself: two halves of a sequence
    fed one after the other reproduce the whole sequence."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w, x = _inputs("bf16", "fwd", 300, d=128)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd")
    d = {k: to_torch(v) for k, v in x.items()}
    state = d["state_in"].clone()
    outs = []
    for lo, hi in ((0, 128), (128, 300)):
        o, s = gdn.forward(d["q"][:, lo:hi].contiguous(), d["k"][:, lo:hi].contiguous(),
                           d["v"][:, lo:hi].contiguous(), d["log_alpha"][:, :, lo:hi].contiguous(),
                           d["beta"][:, :, lo:hi].contiguous(), state, "fwd", state_out=state)
        assert s.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    check(torch.cat(outs, 1).cpu().numpy(), ref, TOL["bf16"], "out (two calls)")
    check(state.cpu().numpy(), ref_s, TOL["bf16"], "state (in place)")


@pytest.mark.parametrize("gate", ["beta0", "no_decay", "forget"])
@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_degenerate_gates(gate, direction):
    w, x = _inputs("f32", direction, 150, state_std=0.3)
    x = dict(x)
    if gate == "beta0":
        x["beta"] = np.zeros_like(x["beta"])
    elif gate == "no_decay":
        x["log_alpha"] = np.zeros_like(x["log_alpha"])
    else:
        x["log_alpha"] = np.full_like(x["log_alpha"], -50.0)
    _compare(x, w)


def test_zero_query_and_key_rows():
    w, x = _inputs("bf16", "bi", 200, d=128)
    x = dict(x)
    q, k = x["q"].copy(), x["k"].copy()
    q[:, 5:9] = 0
    k[:, 40:47] = 0
    q[:, 130] = 0
    k[:, 130] = 0
    x["q"], x["k"] = q, k
    _compare(x, w)


@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_bitwise_repeatable(direction):
    w, x = _inputs("bf16", direction, 333, B=2, d=128)
    o1, s1 = run_gpu(x, direction)
    o2, s2 = run_gpu(x, direction)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_ones_nan_input_finishes_promptly(dtype):
    """An input NaN with every bit set (the pattern a bidirectional scan's
    combine uses for "not written yet") is out of contract, but must not make
    the second visitor of a chunk wait for its bounded poll: first visitors
    store canonical NaNs.  41 chunks, bidirectional; the call returns in well
    under the ~1 s a single expired wait would take, and the outputs the NaN
    reaches are NaN."""
    import time

    import torch

    import gated_delta_rule_scan_amd as gdn
    from gdn_testutil import to_torch

    w = synth.Workload("nan payload", 1, 2, 64 * 40 + 17, 64, 64, dtype, "bi", 3.0, 0.0, 51)
    x = synth.generate(w)
    v = x["v"].copy()
    if dtype == "f32":
        v.view(np.uint32)[0, 100, :, :] = 0xFFFFFFFF
    else:
        v.view(np.uint16)[0, 100, :, :] = 0xFFFF
    d = {k: to_torch(a) for k, a in x.items()}
    d["v"] = to_torch(v)
    gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, "bi")  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out, s = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, "bi")
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert dt < 0.3, f"call took {dt:.3f} s: a combine wait expired"
    o = out.cpu().numpy()
    # the forward memory carries the NaN from token 100 on, the reverse one up to it
    assert np.all(np.isnan(o[0, 100:])) and np.all(np.isnan(o[0, :101]))
