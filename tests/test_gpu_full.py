"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times.  The GPU computes every head; the oracle recomputes a sample
of (batch, head) chains in full (every token and the final state), which is
exactly the oracle restricted to those chains since chains are independent.

Workloads (synth.WORKLOADS): streaming 480p causal rollout (21 calls of 1560
tokens with the state carried in place), 480p bidirectional B2 H16 T32760,
720p causal B1 H16 T75600 with a nonzero initial state, 720p long
bidirectional B1 H24 T111600, and the slow-decay stress variant of the 720p
causal rollout.
"""
import numpy as np
import pytest

import oracle
import synth
from gdn_testutil import TOL, check, check_scaled, rel_err, to_torch

pytestmark = pytest.mark.gpu


def _sample_heads(w):
    hs = [(0, 0), (w.B - 1, w.H - 1), (w.B // 2, w.H // 2)]
    return list(dict.fromkeys(hs))


def run_streaming(d, w, dirs=1):
    """Frame-by-frame calls with the state carried in place (state_in is state_out)."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    T, fr = w.T, w.frame
    out = torch.empty((w.B, T, w.H, w.dv), dtype=torch.float32, device="cuda")
    state = torch.zeros((dirs, w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    if d["state_in"] is not None:
        state.copy_(d["state_in"])
    ws = torch.empty(gdn.workspace_bytes(w.B, fr, w.H, w.dk, w.dv, w.dtype, w.direction), dtype=torch.uint8,
                     device="cuda")
    for f0 in range(0, T, fr):
        f1 = min(T, f0 + fr)
        sl = lambda x: x[:, f0:f1].contiguous()
        gl = lambda x: x[:, :, f0:f1].contiguous()
        o, _ = gdn.forward(sl(d["q"]), sl(d["k"]), sl(d["v"]), gl(d["log_alpha"]), gl(d["beta"]), state, w.direction,
                           out=torch.empty((w.B, f1 - f0, w.H, w.dv), dtype=torch.float32, device="cuda"),
                           state_out=state, workspace=ws)
        out[:, f0:f1] = o
    return out, state


@pytest.mark.parametrize("name", ["stream480", "bidir480", "causal720", "bidir720", "causal720_slow"])
def test_full_size_sampled_heads(name):
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.WORKLOADS[name]
    print(f"\n[{name}] generating {w}", flush=True)
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    print(f"[{name}] GPU run", flush=True)
    if w.frame:
        out, s_out = run_streaming(d, w, w.dirs)
    else:
        out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction)
    torch.cuda.synchronize()
    heads = _sample_heads(w)
    print(f"[{name}] oracle on heads {heads}", flush=True)
    ref, ref_s = oracle.forward_heads(x, heads, w.direction)
    got = np.stack([out[b, :, h].cpu().numpy() for b, h in heads])
    got_s = np.stack([s_out[:, b, h].cpu().numpy() for b, h in heads], axis=1)
    e_o = check(got, ref, TOL[w.dtype], f"{name} out")
    e_s = check(got_s, ref_s, TOL[w.dtype], f"{name} state")
    print(f"[{name}] max|err|/RMS: out {e_o:.3e}  state {e_s:.3e}", flush=True)
    del d, out, s_out
    torch.cuda.empty_cache()


def test_full_size_bidir480_disjoint_regions():
    """The 480p bidirectional workload (B2 H16 T32760) with both directions
    reading before the token's own write, sampled heads against the oracle
    (output bar: the usual factor times the inclusive readout's RMS)."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.WORKLOADS["bidir480"]
    print(f"\n[bidir480 exclusive] generating {w}", flush=True)
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction,
                             exclusive="both")
    torch.cuda.synchronize()
    heads = _sample_heads(w)[:2]
    print(f"[bidir480 exclusive] oracle on heads {heads}", flush=True)
    ref, ref_s = oracle.forward_heads(x, heads, w.direction, exclusive="both")
    ref_incl, _ = oracle.forward_heads(x, heads, w.direction)
    got = np.stack([out[b, :, h].cpu().numpy() for b, h in heads])
    got_s = np.stack([s_out[:, b, h].cpu().numpy() for b, h in heads], axis=1)
    # bar: the inclusive readout's RMS (the exclusive output is a remainder of the same products)
    e_o = check_scaled(got, ref, TOL[w.dtype], float(np.sqrt(np.mean(ref_incl ** 2))), "bidir480 exclusive out")
    e_s = check(got_s, ref_s, TOL[w.dtype], "bidir480 exclusive state")
    print(f"[bidir480 exclusive] max|err|/RMS: out {e_o:.3e}  state {e_s:.3e}", flush=True)
    del d, out, s_out
    torch.cuda.empty_cache()
