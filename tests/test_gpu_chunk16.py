"""16-token chunks on the GPU: parity against the double-precision oracle.

The chunked form is exact at any chunk length ("Video DeltaNet", *Key
Contributions* item 4: chunk-wise scans).  At 16 tokens a chunk's inverse is
one 16 x 16 block and the state advances every 16 tokens; the two-role state
chain runs it, each product's token contraction padded from 16 to 32 with
zeros.  Sizes span many chunks and a ragged tail; the bar is that of every
other chunk length (bf16 inputs: 2e-2 x RMS; fp32 inputs: 1e-4 x RMS).
"""
import numpy as np
import pytest

import oracle
import synth
from gdn_testutil import TOL, check, run_gpu, to_torch

pytestmark = pytest.mark.gpu


def _case(dtype, direction, T, B=1, H=2, dk=64, dv=64, la_shift=3.0, state_std=0.0, seed=0, qk="unit"):
    return synth.Workload("c16", B, H, T, dk, dv, dtype, direction, la_shift, state_std, seed, qk=qk)


def _compare(w, dv_tile=0, **kw):
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], w.direction,
                                erase=kw.get("erase", True), exclusive=kw.get("exclusive", "none"))
    print(f"\n[C=16] {w}", flush=True)
    out, s = run_gpu(x, w.direction, chunk=16, dv_tile=dv_tile, **kw)
    e1 = check(out, ref, TOL[w.dtype], f"out {w} C=16")
    e2 = check(s, ref_s, TOL[w.dtype], f"state {w} C=16")
    print(f"{w.dtype} {w.direction} T={w.T} d={w.dk}/{w.dv} C=16 tile={dv_tile} {kw}: out {e1:.2e} state {e2:.2e}",
          flush=True)
    return out, s


def test_tiny_causal_fp32_chunk16():
    """The tiny causal workload (B1 H2 T256 d64 fp32, sixteen chunks)."""
    _compare(synth.WORKLOADS["tiny"])


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk16_directions_ragged(direction, dtype, d):
    """Every direction and operand type, d = 64 and 128, T = 203 (the last of
    13 chunks ragged), nonzero initial state."""
    _compare(_case(dtype, direction, T=203, H=3, dk=d, dv=d, state_std=0.05, seed=81))


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk16_raw_qk(direction, dtype):
    """q and k not of unit length (per-row scales 1e-3 .. 1e3, rows at the
    norm clamp)."""
    _compare(_case(dtype, direction, T=200, H=3, dk=128, dv=64, state_std=0.05, seed=82, qk="raw"))


@pytest.mark.parametrize("dv_tile", [16, 32])
def test_chunk16_value_tiles(dv_tile):
    _compare(_case("bf16", "bi", T=300, B=2, H=2, dk=128, dv=128, state_std=0.05, seed=83), dv_tile=dv_tile)


def test_chunk16_erase_free_and_slow_decay():
    _compare(_case("bf16", "bi", T=250, H=2, dk=128, dv=128, state_std=0.05, seed=84), erase=False)
    _compare(_case("f32", "bi", T=250, H=2, dk=64, dv=64, la_shift=-2.0, state_std=0.05, seed=85))


@pytest.mark.parametrize("exclusive", ["fwd", "rev", "both"])
def test_chunk16_exclusive_fp32(exclusive):
    _compare(_case("f32", "bi", T=200, H=2, dk=64, dv=64, state_std=0.05, seed=86), exclusive=exclusive)


def test_chunk16_single_token_and_exact_multiple():
    for T in (1, 16, 17, 160):
        _compare(_case("bf16", "bi", T=T, H=2, dk=128, dv=128, state_std=0.05, seed=87))


def test_chunk16_concurrent_matches_serial_and_deterministic():
    """130 chunks on few compute units: the preparation pass beside the
    chain equals the serial order bit for bit, and a repeat equals both."""
    w = _case("bf16", "fwd", T=16 * 129 + 9, H=2, dk=128, dv=128, state_std=0.05, seed=88)
    x = synth.generate(w)
    o_ser, s_ser = run_gpu(x, "fwd", chunk=16, serial=True)
    o_con, s_con = run_gpu(x, "fwd", chunk=16)
    o_rep, s_rep = run_gpu(x, "fwd", chunk=16)
    assert np.array_equal(o_ser, o_con) and np.array_equal(s_ser, s_con)
    assert np.array_equal(o_con, o_rep) and np.array_equal(s_con, s_rep)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd")
    check(o_con, ref, TOL["bf16"], "out concurrent C=16")
    check(s_con, ref_s, TOL["bf16"], "state concurrent C=16")


def test_chunk16_full_size_bidir480_sampled_heads():
    """The 480p bidirectional workload (B2 H16 T32760) at 16-token chunks
    (2048 chunks per direction): sampled (batch, head) chains in full."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.WORKLOADS["bidir480"]
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction, chunk=16)
    torch.cuda.synchronize()
    hs = [(0, 0), (w.B - 1, w.H - 1)]
    ref, ref_s = oracle.forward_heads(x, hs, w.direction)
    got = np.stack([out[b, :, h].cpu().numpy() for b, h in hs])
    got_s = np.stack([s_out[:, b, h].cpu().numpy() for b, h in hs], axis=1)
    e_o = check(got, ref, TOL[w.dtype], "bidir480 C=16 out")
    e_s = check(got_s, ref_s, TOL[w.dtype], "bidir480 C=16 state")
    print(f"\n[bidir480 C=16] max|err|/RMS: out {e_o:.3e}  state {e_s:.3e}", flush=True)
    del d, out, s_out
    torch.cuda.empty_cache()
