"""GPU parity of the frame-wise delta operator (gdn_vda_forward) against its
double-precision oracle (oracle/vda.py), element by element over every output
and final state, at the tolerances of tests/gdn_testutil.py (bf16 inputs
2e-2 x RMS, fp32 inputs 1e-4 x RMS).

Small cases cover fp32 and bf16, all directions, dk/dv in {64, 128}, frames of
1, 16, 30, 100 and 200 tokens with ragged ends, with and without an initial
state; the full-size case is the 480p bidirectional shape (B2 H16, 21 frames
of 1560 tokens) with the oracle on sampled heads.
"""
import numpy as np
import pytest

import synth
from gdn_testutil import TOL, check, to_torch
from oracle import vda as vda_oracle

pytestmark = pytest.mark.gpu


def _workload(dtype, direction, T, frame, B=1, H=2, dk=64, dv=64, std=0.05, seed=21, shift=-3.0):
    w = synth.Workload("vda", B, H, T, dk, dv, dtype, direction, shift, std, seed)
    return w, synth.generate_frames(w, frame)


def _run(x, direction, frame, want_state=True, state_in="use", write="inverse", lag=0, epi=None):
    import torch

    import gated_delta_rule_scan_amd as gdn

    d = {k: to_torch(v) for k, v in x.items()}
    s_in = d["state_in"] if state_in == "use" else state_in
    ekw = {}
    if epi is not None:
        ekw = dict(gate=to_torch(epi["gate"]), norm_weight=to_torch(epi["norm_weight"]), norm_eps=epi["eps"])
    out, s = gdn.vda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s_in, direction, frame,
                             want_state=want_state, write=write, lag=lag, **ekw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if s is None else s.cpu().numpy())


def _compare(dtype, direction, T, frame, write="inverse", lag=0, epilogue=False, **kw):
    w, x = _workload(dtype, direction, T, frame, **kw)
    epi = None
    okw = {}
    if epilogue:
        epi = dict(synth.generate_epilogue(w), eps=1e-6)
        okw = dict(gate=epi["gate"], norm_weight=epi["norm_weight"], norm_eps=1e-6)
    ref, ref_s = vda_oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction, frame,
                                    write=write, lag=lag, **okw)
    out, s = _run(x, direction, frame, write=write, lag=lag, epi=epi)
    tag = f"{w} frame={frame} write={write} lag={lag} epilogue={epilogue}"
    e1 = check(out, ref, TOL[dtype], f"vda out {tag}")
    e2 = check(s, ref_s, TOL[dtype], f"vda state {tag}")
    print(f"\nvda {dtype} {direction} T={T} frame={frame} d={w.dk}/{w.dv} {write} lag={lag} epi={int(epilogue)}: "
          f"out {e1:.2e} state {e2:.2e}", flush=True)


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_directions(dtype, direction):
    _compare(dtype, direction, T=333, frame=100, H=3)


@pytest.mark.parametrize("frame", [1, 16, 30, 200])
def test_frame_sizes(frame):
    _compare("f32", "bi", T=150 if frame > 1 else 40, frame=frame)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head_dims(dk, dv, dtype):
    _compare(dtype, "bi", T=260, frame=64, dk=dk, dv=dv, seed=22)


def test_no_initial_state_and_fast_decay():
    _compare("bf16", "fwd", T=300, frame=64, std=0.0, shift=3.0, dk=128, dv=128)


def test_empty_sequence_passes_state_through():
    import torch

    import gated_delta_rule_scan_amd as gdn

    rng = np.random.default_rng(3)
    s_in = rng.standard_normal((2, 1, 2, 64, 64)).astype(np.float32)
    e = torch.empty((1, 0, 2, 64), dtype=torch.bfloat16, device="cuda")
    la = torch.empty((2, 1, 0, 2), dtype=torch.float32, device="cuda")
    out, s = gdn.vda_forward(e, e, e, la, la, to_torch(s_in), "bi", 16)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (1, 0, 2, 64) and np.array_equal(s.cpu().numpy(), s_in)


def test_bitwise_repeatable():
    w, x = _workload("bf16", "bi", 500, 128, dk=128, dv=128)
    o1, s1 = _run(x, "bi", 128)
    o2, s2 = _run(x, "bi", 128)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_full_size_480p_bidirectional_sampled_heads():
    """B2 H16 d128 bf16, 21 frames of 1560 tokens (30 x 52 latent), both directions;
    the oracle recomputes three (batch, head) chains over every token."""
    w = synth.Workload("vda480", 2, 16, 32760, 128, 128, "bf16", "bi", -3.0, 0.0, 2)
    x = synth.generate_frames(w, 1560)
    out, s = _run(x, "bi", 1560)
    for b, h in [(0, 0), (1, 15), (1, 8)]:
        sel = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v")}
        la = x["log_alpha"][:, b:b + 1, :, h:h + 1]
        bt = x["beta"][:, b:b + 1, :, h:h + 1]
        ref, ref_s = vda_oracle.forward(sel["q"], sel["k"], sel["v"], la, bt, None, "bi", 1560)
        e1 = check(out[b:b + 1, :, h:h + 1], ref, TOL["bf16"], f"vda480 out b{b} h{h}")
        e2 = check(s[:, b:b + 1, h:h + 1], ref_s, TOL["bf16"], f"vda480 state b{b} h{h}")
        print(f"\nvda480 b{b} h{h}: out {e1:.2e} state {e2:.2e}", flush=True)


# ---- additive frame writes, readout lag, epilogue ----

@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_additive_write(dtype, direction):
    _compare(dtype, direction, T=333, frame=100, H=3, write="additive")


@pytest.mark.parametrize("frame", [1, 30])
def test_additive_write_frame_sizes(frame):
    _compare("f32", "bi", T=150 if frame > 1 else 40, frame=frame, write="additive", dk=128, dv=64)


@pytest.mark.parametrize("lag", [1, 2, 5])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_readout_lag(dtype, lag):
    # ragged last frame; the initial states are read near the edges
    _compare(dtype, "bi", T=290, frame=64, lag=lag, dk=128, dv=128, seed=23)


def test_readout_lag_single_direction_without_initial_state():
    _compare("bf16", "rev", T=200, frame=30, lag=2, std=0.0, seed=24)
    _compare("bf16", "fwd", T=200, frame=30, lag=3, std=0.0, seed=25)


@pytest.mark.parametrize("direction", ["fwd", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_epilogue(dtype, direction):
    _compare(dtype, direction, T=260, frame=64, epilogue=True, dk=128, dv=128, seed=26)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_epilogue_with_lag_and_additive_write(dk, dv):
    _compare("bf16", "bi", T=300, frame=50, epilogue=True, lag=2, write="additive", dk=dk, dv=dv, seed=27)


def test_full_size_480p_disjoint_regions_with_epilogue():
    """B2 H16 d128 bf16, 21 frames of 1560 tokens, both directions, a 15-frame
    local window (readout lag 8), text state S_T/2 in each direction, and the
    RMS-norm plus gate epilogue; the oracle recomputes two sampled heads."""
    import numpy as np

    w = synth.Workload("vda480", 2, 16, 32760, 128, 128, "bf16", "bi", -3.0, 0.0, 2)
    x = synth.generate_frames(w, 1560)
    S_T = synth.normals(5, 70, (2, 16, 128, 128), 0.05)
    x["state_in"] = np.ascontiguousarray(np.stack([S_T / 2, S_T / 2]).astype(np.float32))
    epi = dict(synth.generate_epilogue(w), eps=1e-6)
    out, s = _run(x, "bi", 1560, lag=8, epi=epi)
    for b, h in [(0, 3), (1, 12)]:
        sel = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v")}
        ref, ref_s = vda_oracle.forward(sel["q"], sel["k"], sel["v"], x["log_alpha"][:, b:b + 1, :, h:h + 1],
                                        x["beta"][:, b:b + 1, :, h:h + 1], x["state_in"][:, b:b + 1, h:h + 1], "bi",
                                        1560, lag=8, gate=epi["gate"][b:b + 1, :, h:h + 1],
                                        norm_weight=epi["norm_weight"], norm_eps=1e-6)
        e1 = check(out[b:b + 1, :, h:h + 1], ref, TOL["bf16"], f"vda480 lag8 epi out b{b} h{h}")
        e2 = check(s[:, b:b + 1, h:h + 1], ref_s, TOL["bf16"], f"vda480 lag8 epi state b{b} h{h}")
        print(f"\nvda480 lag8 epilogue b{b} h{h}: out {e1:.2e} state {e2:.2e}", flush=True)


def test_full_size_720p_bidirectional_sampled_heads():
    """B1 H24 d128 bf16, 31 frames of 3600 tokens (45 x 80 latent), both
    directions; the oracle recomputes two sampled heads over every token."""
    w = synth.Workload("vda720", 1, 24, 111600, 128, 128, "bf16", "bi", -3.0, 0.0, 4)
    x = synth.generate_frames(w, 3600)
    out, s = _run(x, "bi", 3600)
    for b, h in [(0, 0), (0, 23)]:
        sel = {n: x[n][b:b + 1, :, h:h + 1] for n in ("q", "k", "v")}
        ref, ref_s = vda_oracle.forward(sel["q"], sel["k"], sel["v"], x["log_alpha"][:, b:b + 1, :, h:h + 1],
                                        x["beta"][:, b:b + 1, :, h:h + 1], None, "bi", 3600)
        e1 = check(out[b:b + 1, :, h:h + 1], ref, TOL["bf16"], f"vda720 out b{b} h{h}")
        e2 = check(s[:, b:b + 1, h:h + 1], ref_s, TOL["bf16"], f"vda720 state b{b} h{h}")
        print(f"\nvda720 b{b} h{h}: out {e1:.2e} state {e2:.2e}", flush=True)
