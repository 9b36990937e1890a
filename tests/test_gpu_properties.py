"""Properties of the scan that hold at any size, checked on the GPU between
calls of the library itself (no oracle on the compared side):

* the reverse scan is the forward scan of the token-reversed sequence
  (flip . forward . flip), with its own gates and initial state;
* the bidirectional scan is the sum of a forward and a reverse scan, each
  with its own gates and initial state ("Video DeltaNet", *Methodology in
  Plain English*: a forward and a backward recurrent state whose readouts
  are added);
* the scan is linear in (initial state, v) jointly: S_t = a_t S_{t-1} (I -
  b_t k_t k_t^T) + b_t v_t k_t^T and o_t = S_t q_t.

The oracle pins the same properties on the CPU (tests/test_oracle_pins.py);
here they check the kernels' own paths against each other, at sizes with a
ragged last chunk.
"""
import numpy as np
import pytest

import synth
from gdn_testutil import TOL, rel_err, run_gpu

pytestmark = pytest.mark.gpu


def _inputs(dtype, direction, T=333, H=3, d=64, seed=71):
    w = synth.Workload("prop", 1, H, T, d, d, dtype, direction, 3.0, 0.05, seed)
    return w, synth.generate(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reverse_is_flipped_forward(dtype):
    """rev(x) == flip(fwd(flip(x))): the two runs see different chunk
    boundaries (T = 333 is no multiple of 64), so they agree to the bar, not
    bit for bit."""
    w, x = _inputs(dtype, "rev")
    out_r, s_r = run_gpu(x, "rev")
    f = {k: (None if v is None else v) for k, v in x.items()}
    f["q"], f["k"], f["v"] = (np.ascontiguousarray(x[n][:, ::-1]) for n in ("q", "k", "v"))
    f["log_alpha"] = np.ascontiguousarray(x["log_alpha"][:, :, ::-1])
    f["beta"] = np.ascontiguousarray(x["beta"][:, :, ::-1])
    out_f, s_f = run_gpu(f, "fwd")
    e_o, _, _ = rel_err(out_r, out_f[:, ::-1])
    e_s, _, _ = rel_err(s_r, s_f)
    print(f"\n{dtype}: reverse against flipped forward: out {e_o:.2e} state {e_s:.2e} x RMS", flush=True)
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidirectional_is_forward_plus_reverse(dtype):
    """bi(x) == fwd(x) + rev(x), each direction with its own gates and
    initial state, bit for bit; the final states are the two directions'
    own."""
    w, x = _inputs(dtype, "bi")
    out_b, s_b = run_gpu(x, "bi")
    parts = []
    for slot, direction in ((0, "fwd"), (1, "rev")):
        y = dict(x)
        y["log_alpha"] = np.ascontiguousarray(x["log_alpha"][slot:slot + 1])
        y["beta"] = np.ascontiguousarray(x["beta"][slot:slot + 1])
        y["state_in"] = np.ascontiguousarray(x["state_in"][slot:slot + 1])
        parts.append(run_gpu(y, direction))
    summed = parts[0][0] + parts[1][0]
    states = np.concatenate([parts[0][1], parts[1][1]], axis=0)
    e_o, _, _ = rel_err(out_b, summed)
    e_s, _, _ = rel_err(s_b, states)
    print(f"\n{dtype}: bidirectional against forward + reverse: out {e_o:.2e} state {e_s:.2e} x RMS "
          f"(bitwise: {np.array_equal(out_b, summed)}, {np.array_equal(s_b, states)})", flush=True)
    # each direction's readout and state come from the same arithmetic in
    # both launch shapes, and the second visitor of a chunk adds the first
    # one's readout once (an fp32 addition, commutative): bit for bit
    assert np.array_equal(out_b, summed) and np.array_equal(s_b, states)


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
def test_linear_in_state_and_values(direction):
    """fp32: scan(s1 + 2 s2, v1 + 2 v2) == scan(s1, v1) + 2 scan(s2, v2),
    outputs and final states, with q, k and the gates shared."""
    w, x1 = _inputs("f32", direction, seed=72)
    _, x2 = _inputs("f32", direction, seed=73)
    x2 = dict(x2, q=x1["q"], k=x1["k"], log_alpha=x1["log_alpha"], beta=x1["beta"])
    xs = dict(x1, v=x1["v"] + 2 * x2["v"], state_in=x1["state_in"] + 2 * x2["state_in"])
    o1, s1 = run_gpu(x1, direction)
    o2, s2 = run_gpu(x2, direction)
    os_, ss = run_gpu(xs, direction)
    e_o, _, _ = rel_err(os_, o1 + 2 * o2)
    e_s, _, _ = rel_err(ss, s1 + 2 * s2)
    print(f"\n{direction}: linearity in (state_in, v): out {e_o:.2e} state {e_s:.2e} x RMS", flush=True)
    assert e_o <= TOL["f32"] and e_s <= TOL["f32"]
