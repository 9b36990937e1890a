"""Memory discipline of the library calls on the GPU:

* poisoned outputs and workspace -- `out`, `state_out` and the workspace are
  filled with all-ones bytes (a NaN pattern) before the call; the results must
  equal, bit for bit, a call on zero-filled buffers (every output element is
  written, and no unwritten workspace byte is read);
* guard canaries -- every buffer, inputs included, sits inside a larger
  allocation with 4 KiB guard zones of a known byte pattern on both sides; the
  zones must be intact after the call (no access writes out of bounds);
* a streaming rollout (several calls, the state carried in place) captured as
  one HIP graph and replayed, equal to the eager rollout;
* a starved preparation pass (forced from the host with a test-only option):
  the state chain's bounded waits expire and every result is NaN.
"""
import numpy as np
import pytest

import synth
from gdn_testutil import to_torch

pytestmark = pytest.mark.gpu

G = 4096  # guard bytes on each side


def _guarded(t, pattern):
    """Copy of tensor t inside a guarded uint8 allocation; returns (view, whole)."""
    import torch

    n = t.numel() * t.element_size()
    whole = torch.full((n + 2 * G,), pattern, dtype=torch.uint8, device="cuda")
    view = whole[G:G + n].view(t.dtype).view(t.shape)
    view.copy_(t)
    return view, whole


def _guards_intact(whole, pattern):
    import torch

    return bool(torch.all(whole[:G] == pattern)) and bool(torch.all(whole[-G:] == pattern))


def _token_call(x, direction, fill, guard=False):
    import torch

    import gated_delta_rule_scan_amd as gdn

    d = {k: to_torch(v) for k, v in x.items()}
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    dirs = 2 if direction == "bi" else 1
    prob = gdn.gdn_problem_t(B=B, T=T, H=H, dk=dk, dv=dv,
                             dtype=gdn.GDN_DTYPE_BF16 if d["q"].dtype == torch.bfloat16 else gdn.GDN_DTYPE_F32)
    nws = gdn.gdn_workspace_bytes(prob, gdn.DIRECTIONS[direction])
    out = torch.full((B, T, H, dv), 0, dtype=torch.float32, device="cuda")
    s_out = torch.full((dirs, B, H, dv, dk), 0, dtype=torch.float32, device="cuda")
    ws = torch.full((nws,), 0, dtype=torch.uint8, device="cuda")
    for t in (out, s_out, ws):
        t.view(torch.uint8).fill_(fill)
    wholes = []
    if guard:
        for k in [k for k in d if d[k] is not None]:
            d[k], wh = _guarded(d[k], 0x5A)
            wholes.append(wh)
        out, wo = _guarded(out, 0x5A)
        s_out, wso = _guarded(s_out, 0x5A)
        ws, wws = _guarded(ws, 0x5A)
        wholes += [wo, wso, wws]
    gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], direction, out=out,
                state_out=s_out, workspace=ws)
    torch.cuda.synchronize()
    return out.clone(), s_out.clone(), wholes


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
def test_token_scan_poisoned_buffers(direction):
    import torch

    w = synth.Workload("poison", 2, 3, 700, 128, 64, "bf16", direction, 3.0, 0.02, 51)
    x = synth.generate(w)
    o0, s0, _ = _token_call(x, direction, 0x00)
    o1, s1, _ = _token_call(x, direction, 0xFF)
    assert torch.isfinite(o1).all() and torch.isfinite(s1).all()
    assert torch.equal(o0, o1) and torch.equal(s0, s1)


@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_token_scan_guard_canaries(direction):
    w = synth.Workload("guard", 1, 2, 333, 64, 128, "f32", direction, 3.0, 0.02, 52)
    x = synth.generate(w)
    _, _, wholes = _token_call(x, direction, 0x00, guard=True)
    assert all(_guards_intact(wh, 0x5A) for wh in wholes)


def _vda_call(x, e, direction, frame, fill, guard=False, **kw):
    import torch

    import gated_delta_rule_scan_amd as gdn

    d = {k: to_torch(v) for k, v in x.items()}
    if e is not None:
        d["gate"], d["nw"] = to_torch(e["gate"]), to_torch(e["norm_weight"])
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    dirs = 2 if direction == "bi" else 1
    prob = gdn.gdn_vda_problem_t(B=B, T=T, H=H, dk=dk, dv=dv, frame=frame,
                                 dtype=gdn.GDN_DTYPE_BF16 if d["q"].dtype == torch.bfloat16 else gdn.GDN_DTYPE_F32)
    nws = gdn.gdn_vda_workspace_bytes(prob, gdn.DIRECTIONS[direction])
    out = torch.empty((B, T, H, dv), dtype=torch.float32, device="cuda")
    s_out = torch.empty((dirs, B, H, dv, dk), dtype=torch.float32, device="cuda")
    ws = torch.empty((nws,), dtype=torch.uint8, device="cuda")
    for t in (out, s_out, ws):
        t.view(torch.uint8).fill_(fill)
    wholes = []
    if guard:
        for k in [k for k in d if d[k] is not None]:
            d[k], wh = _guarded(d[k], 0x3C)
            wholes.append(wh)
        out, wo = _guarded(out, 0x3C)
        s_out, wso = _guarded(s_out, 0x3C)
        ws, wws = _guarded(ws, 0x3C)
        wholes += [wo, wso, wws]
    ekw = {} if e is None else dict(gate=d["gate"], norm_weight=d["nw"], norm_eps=1e-6)
    gdn.vda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], direction, frame, out=out,
                    state_out=s_out, workspace=ws, **ekw, **kw)
    torch.cuda.synchronize()
    return out.clone(), s_out.clone(), wholes


@pytest.mark.parametrize("write,lag,epi", [("inverse", 0, False), ("additive", 2, True)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_frame_wise_poisoned_buffers(dtype, write, lag, epi):
    import torch

    w = synth.Workload("poison vda", 2, 2, 450, 64, 128, dtype, "bi", -3.0, 0.05, 53)
    x = synth.generate_frames(w, 64)
    e = synth.generate_epilogue(w) if epi else None
    o0, s0, _ = _vda_call(x, e, "bi", 64, 0x00, write=write, lag=lag)
    o1, s1, _ = _vda_call(x, e, "bi", 64, 0xFF, write=write, lag=lag)
    assert torch.isfinite(o1).all() and torch.isfinite(s1).all()
    assert torch.equal(o0, o1) and torch.equal(s0, s1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_frame_wise_guard_canaries(dtype):
    w = synth.Workload("guard vda", 1, 2, 333, 128, 64, dtype, "bi", -3.0, 0.05, 54)
    x = synth.generate_frames(w, 50)
    e = synth.generate_epilogue(w)
    _, _, wholes = _vda_call(x, e, "bi", 50, 0x00, guard=True, lag=1)
    assert all(_guards_intact(wh, 0x3C) for wh in wholes)


def test_streaming_rollout_graph():
    """Four calls of 300 tokens, the state carried in place, captured as one graph."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.Workload("stream graph", 1, 3, 1200, 128, 128, "bf16", "fwd", 3.0, 0.02, 55)
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    n = 4
    parts = [{k: (d[k][:, 300 * i:300 * (i + 1)].contiguous() if k in ("q", "k", "v") else
                  d[k][:, :, 300 * i:300 * (i + 1)].contiguous()) for k in ("q", "k", "v", "log_alpha", "beta")}
             for i in range(n)]
    outs = [torch.empty((1, 300, 3, 128), dtype=torch.float32, device="cuda") for _ in range(n)]
    state = torch.empty_like(d["state_in"])
    prob = gdn.gdn_problem_t(B=1, T=300, H=3, dk=128, dv=128, dtype=gdn.GDN_DTYPE_BF16)
    ws = torch.empty(gdn.gdn_workspace_bytes(prob, gdn.GDN_DIR_FORWARD), dtype=torch.uint8, device="cuda")

    def rollout():
        for i in range(n):
            gdn.forward(parts[i]["q"], parts[i]["k"], parts[i]["v"], parts[i]["log_alpha"], parts[i]["beta"], state,
                        "fwd", out=outs[i], state_out=state, workspace=ws)

    # eager reference
    state.copy_(d["state_in"])
    rollout()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs] + [state.clone()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        state.copy_(d["state_in"])
        rollout()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rollout()
    for rep in range(3):
        state.copy_(d["state_in"])
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip([o for o in outs] + [state], ref):
            assert torch.equal(a, b), f"replay {rep}"


@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_starved_preparation_gives_nan_not_wrong_results(direction):
    """GDN_OPT_TEST_NO_PREPARATION: the chunk preparation pass is not launched,
    so the state chain's ready flags never clear.  Its bounded waits expire
    and every output and final state is the canonical NaN (not the "not
    written yet" pattern), instead of results computed from a stale
    workspace.  A normal call afterwards is unaffected."""
    import torch

    import gated_delta_rule_scan_amd as gdn
    import oracle
    from gdn_testutil import TOL, check

    w = synth.Workload("starved", 1, 2, 64 * 20 + 5, 64, 64, "bf16", direction, 3.0, 0.05, 41)
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    out = torch.zeros((w.B, w.T, w.H, w.dv), dtype=torch.float32, device="cuda")
    s_out = torch.zeros((w.dirs, w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    dirn = gdn.DIRECTIONS[direction]
    prob = gdn.make_problem(w.B, w.T, w.H, w.dk, w.dv, gdn.GDN_DTYPE_BF16)
    ws = torch.empty(gdn.gdn_workspace_bytes(prob, dirn), dtype=torch.uint8, device="cuda")
    prob.workspace, prob.workspace_bytes = ws.data_ptr(), ws.numel()
    prob.stream = torch.cuda.current_stream().cuda_stream
    prob.options = gdn.GDN_OPT_TEST_NO_PREPARATION
    st = gdn.gdn_forward(prob, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["log_alpha"].data_ptr(),
                         d["beta"].data_ptr(), d["state_in"].data_ptr(), s_out.data_ptr(), out.data_ptr(), dirn)
    assert st == gdn.GDN_OK
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all()) and bool(torch.isnan(s_out).all())
    assert bool((out.view(torch.int32) != -1).all())  # never the all-ones fill pattern
    o2, s2 = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], direction, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction)
    check(o2.cpu().numpy(), ref, TOL["bf16"], "out after the starved call")
    check(s2.cpu().numpy(), ref_s, TOL["bf16"], "state after the starved call")
