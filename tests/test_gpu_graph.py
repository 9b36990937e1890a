"""HIP graph capture of the library calls (the streaming use case asks for it:
"Explore linear attention", "Open questions and risks").  One call is captured
with torch.cuda.graph after an eager warm-up (which creates the library's side
stream and events); the graph is then replayed several times with new inputs
copied in eagerly between replays, and every replay must equal an eager call
on the same inputs bit for bit (the kernels are deterministic).

The token scan is captured with and without GDN_OPT_SERIAL; the shapes below
have 16 or more chunks and few chain workgroups, so an eager call takes the
concurrent preparation path when `serial` is off, while a captured call takes
the serial order (the library checks the stream's capture status).  A first
call of the process made inside a capture is checked in a fresh process."""
import os
import subprocess
import sys

import numpy as np
import pytest

import synth
from gdn_testutil import to_torch

pytestmark = pytest.mark.gpu


def _replays(fn_eager, fn_capture, inputs, fresh, n=3):
    """inputs: dict of static device tensors; fresh(i) -> dict of numpy arrays
    for replay i.  fn_eager(inputs) -> tuple of tensors; fn_capture(inputs)
    captured once."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn_capture(inputs)  # warm-up: creates the library's side stream and events
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn_capture(inputs)
    for i in range(n):
        for k, v in fresh(i).items():
            inputs[k].copy_(to_torch(v))
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        # eager work of the program's own between replays
        want = fn_eager(inputs)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a, b), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("serial", [True, False])
@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_token_scan_capture(direction, serial):
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.Workload("graph", 1, 2, 1100, 128, 128, "bf16", direction, 3.0, 0.02, 31)
    x = synth.generate(w)
    inp = {k: to_torch(v) for k, v in x.items()}
    out = torch.empty((1, 1100, 2, 128), dtype=torch.float32, device="cuda")
    s_out = torch.empty((w.dirs, 1, 2, 128, 128), dtype=torch.float32, device="cuda")
    prob = gdn.gdn_problem_t(B=1, T=1100, H=2, dk=128, dv=128, dtype=gdn.GDN_DTYPE_BF16)
    ws = torch.empty(gdn.gdn_workspace_bytes(prob, gdn.DIRECTIONS[direction]), dtype=torch.uint8, device="cuda")

    def run(d, o=out, so=s_out):
        gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], direction, out=o,
                    state_out=so, workspace=ws, serial=serial)
        return o, so

    def eager(d):
        o = torch.empty_like(out)
        so = torch.empty_like(s_out)
        return run(d, o, so)

    def fresh(i):
        y = synth.generate(w.replace(seed=100 + i))
        return {k: y[k] for k in ("q", "k", "v", "log_alpha", "beta", "state_in")}

    _replays(eager, run, inp, fresh)


@pytest.mark.parametrize("lag,epilogue", [(0, False), (2, True)])
def test_frame_wise_capture(lag, epilogue):
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.Workload("graph vda", 1, 2, 900, 128, 128, "bf16", "bi", -3.0, 0.05, 32)
    x = synth.generate_frames(w, 100)
    inp = {k: to_torch(v) for k, v in x.items()}
    ekw = {}
    if epilogue:
        e = synth.generate_epilogue(w)
        inp["gate"] = to_torch(e["gate"])
        ekw = dict(norm_weight=to_torch(e["norm_weight"]), norm_eps=1e-6)
    out = torch.empty((1, 900, 2, 128), dtype=torch.float32, device="cuda")
    s_out = torch.empty((2, 1, 2, 128, 128), dtype=torch.float32, device="cuda")
    prob = gdn.gdn_vda_problem_t(B=1, T=900, H=2, dk=128, dv=128, frame=100, dtype=gdn.GDN_DTYPE_BF16)
    ws = torch.empty(gdn.gdn_vda_workspace_bytes(prob, gdn.GDN_DIR_BIDIRECTIONAL), dtype=torch.uint8, device="cuda")

    def run(d, o=out, so=s_out):
        gdn.vda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], "bi", 100, out=o,
                        state_out=so, workspace=ws, lag=lag, gate=d.get("gate"), **ekw)
        return o, so

    def eager(d):
        return run(d, torch.empty_like(out), torch.empty_like(s_out))

    def fresh(i):
        y = synth.generate_frames(w.replace(seed=200 + i), 100)
        f = {k: y[k] for k in ("q", "k", "v", "log_alpha", "beta", "state_in")}
        if epilogue:
            f["gate"] = synth.generate_epilogue(w.replace(seed=200 + i))["gate"]
        return f

    _replays(eager, run, inp, fresh)


_FIRST_CALL_IN_CAPTURE = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + '/tests')
import synth, gated_delta_rule_scan_amd as gdn
from gdn_testutil import to_torch
w = synth.Workload("graph first", 1, 2, 1100, 128, 128, "bf16", "bi", 3.0, 0.02, 33)
inp = {k: to_torch(v) for k, v in synth.generate(w).items()}
out = torch.empty((1, 1100, 2, 128), dtype=torch.float32, device="cuda")
s_out = torch.empty((2, 1, 2, 128, 128), dtype=torch.float32, device="cuda")
prob = gdn.gdn_problem_t(B=1, T=1100, H=2, dk=128, dv=128, dtype=gdn.GDN_DTYPE_BF16)
ws = torch.empty(gdn.gdn_workspace_bytes(prob, gdn.GDN_DIR_BIDIRECTIONAL), dtype=torch.uint8, device="cuda")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g):  # the first library call of this process
    gdn.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["state_in"], "bi", out=out,
                state_out=s_out, workspace=ws)
for i in range(3):
    y = synth.generate(w.replace(seed=300 + i))
    for k in ("q", "k", "v", "log_alpha", "beta", "state_in"):
        inp[k].copy_(to_torch(y[k]))
    g.replay()
    torch.cuda.synchronize()
    got = (out.clone(), s_out.clone())
    o2, s2 = gdn.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["state_in"], "bi")
    torch.cuda.synchronize()
    assert torch.equal(got[0], o2) and torch.equal(got[1], s2), f"replay {i} differs from the eager call"
print("FIRST_CALL_IN_CAPTURE_OK", flush=True)
"""


def test_first_call_of_the_process_inside_a_capture():
    """A fresh process whose first library call is captured (no eager warm-up
    has created the library's side stream): the capture takes the serial
    order, and each of three replays with new inputs equals an eager call
    bit for bit."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_IN_CAPTURE, root], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and "FIRST_CALL_IN_CAPTURE_OK" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]


def test_call_on_a_non_current_stream_keeps_its_buffers():
    """forward(stream=s) with s not the current stream: the workspace and
    outputs the binding allocates are recorded on s, so memory allocated
    right after the call on the current stream (and written at once) never
    lands in a buffer the scan still uses; the result equals a call on the
    current stream bit for bit."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.Workload("stream", 2, 8, 64 * 60 + 9, 128, 128, "bf16", "bi", 3.0, 0.02, 34)
    inp = {k: to_torch(v) for k, v in synth.generate(w).items()}
    ref_o, ref_s = gdn.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["state_in"], "bi")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        o, s = gdn.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["state_in"], "bi",
                           stream=side)
        # new allocations on the current stream, written at once
        junk = [torch.full((1 << 22,), float("nan"), device="cuda") for _ in range(16)]
        torch.cuda.current_stream().wait_stream(side)
        assert torch.equal(o, ref_o) and torch.equal(s, ref_s)
        del junk, o, s
