"""128-token chunks on the GPU: parity against the double-precision oracle and
invariance of the output and final states to the chunk length.

The chunked form evaluates the recurrence exactly at any chunk length
("Video DeltaNet", *Key Contributions* item 4: chunk-wise scans), so every
chunk length must reach the oracle within the stated bar (bf16 inputs: 2e-2 x
RMS; fp32 inputs: 1e-4 x RMS).  At 128 tokens the chunk preparation is its own
kernel (the blocked fp32 inverse of a 128 x 128 unit triangle) and the state
chain is the two-role chain with two token row tiles per wave.  Sizes span
several chunks and a ragged tail (T mod 128 != 0).
"""
import numpy as np
import pytest

import oracle
import synth
from gdn_testutil import TOL, check, rel_err, run_gpu, to_torch

pytestmark = pytest.mark.gpu


def _case(dtype, direction, T, B=1, H=2, dk=64, dv=64, la_shift=3.0, state_std=0.0, seed=0, qk="unit"):
    return synth.Workload("c128", B, H, T, dk, dv, dtype, direction, la_shift, state_std, seed, qk=qk)


def _compare(w, chunk=128, dv_tile=0, **kw):
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], w.direction,
                                erase=kw.get("erase", True), exclusive=kw.get("exclusive", "none"))
    print(f"\n[C={chunk}] {w}", flush=True)
    out, s = run_gpu(x, w.direction, chunk=chunk, dv_tile=dv_tile, **kw)
    e1 = check(out, ref, TOL[w.dtype], f"out {w} C={chunk}")
    e2 = check(s, ref_s, TOL[w.dtype], f"state {w} C={chunk}")
    print(f"{w.dtype} {w.direction} T={w.T} d={w.dk}/{w.dv} C={chunk} tile={dv_tile} {kw}: out {e1:.2e} state {e2:.2e}",
          flush=True)
    return out, s


def test_tiny_causal_fp32_chunk128():
    """The tiny causal workload (B1 H2 T256 d64 fp32, two whole chunks)."""
    _compare(synth.WORKLOADS["tiny"])


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_chunk128_directions_ragged(direction, dtype, d):
    """Every direction and operand type, d = 64 and 128, T = 333 (three chunks,
    the last one ragged), nonzero initial state."""
    _compare(_case(dtype, direction, T=333, H=3, dk=d, dv=d, state_std=0.05, seed=31))


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk128_raw_qk(direction, dtype):
    """q and k not of unit length (per-row scales 1e-3 .. 1e3, rows at the
    norm clamp): the 128-token preparation's own row scales."""
    _compare(_case(dtype, direction, T=300, H=3, dk=128, dv=64, state_std=0.05, seed=32, qk="raw"))


@pytest.mark.parametrize("dv_tile", [16, 32])
def test_chunk128_value_tiles_bf16(dv_tile):
    """Both value-tile widths of the bf16 chain at 128-token chunks."""
    _compare(_case("bf16", "bi", T=400, B=2, H=2, dk=128, dv=128, state_std=0.05, seed=33), dv_tile=dv_tile)


@pytest.mark.parametrize("la_shift", [3.0, -2.0])
def test_chunk128_decay_regimes(la_shift):
    """Fast decay (log-gate sums of several hundred inside a chunk, many decay
    factors below fp32's range) and slow decay (long-range state)."""
    _compare(_case("f32", "bi", T=390, H=2, dk=64, dv=64, la_shift=la_shift, state_std=0.05, seed=34))


def test_chunk128_erase_free():
    """The erase-free variant (L = 0, so the inverse is the identity)."""
    _compare(_case("bf16", "bi", T=300, H=2, dk=128, dv=128, state_std=0.05, seed=35), erase=False)


@pytest.mark.parametrize("exclusive", ["fwd", "rev", "both"])
def test_chunk128_exclusive_fp32(exclusive):
    """Exclusive readouts on fp32 operands (the bf16 ones need the low parts
    the column chain carries, so 128-token chunks reject them)."""
    _compare(_case("f32", "bi", T=300, H=2, dk=64, dv=64, state_std=0.05, seed=36), exclusive=exclusive)


def test_chunk128_single_token_and_exact_multiple():
    """A one-token sequence and an exact multiple of the chunk length."""
    for T in (1, 256):
        _compare(_case("bf16", "bi", T=T, H=2, dk=128, dv=128, state_std=0.05, seed=37))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_length_invariance(dtype):
    """The same inputs at chunk lengths 16, 32, 64 and 128: every output and
    final state within the bar of the oracle, and of each other (the chunked
    form is exact, so only rounding may differ between chunk lengths)."""
    w = _case(dtype, "bi", T=520, H=2, dk=128, dv=128, state_std=0.05, seed=38)
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi")
    runs = {}
    for C in (16, 32, 64, 128):
        out, s = run_gpu(x, "bi", chunk=C)
        check(out, ref, TOL[dtype], f"out C={C}")
        check(s, ref_s, TOL[dtype], f"state C={C}")
        runs[C] = (out, s)
    for C in (16, 32, 64):
        e_o, _, _ = rel_err(runs[128][0], runs[C][0])
        e_s, _, _ = rel_err(runs[128][1], runs[C][1])
        print(f"\n{dtype}: C=128 against C={C}: out {e_o:.2e} state {e_s:.2e} x RMS", flush=True)
        assert e_o <= TOL[dtype] and e_s <= TOL[dtype]


def test_chunk128_concurrent_matches_serial():
    """20 chunks of one direction with a chain on few compute units: the
    preparation pass runs beside the chain, which waits on per-chunk ready
    flags; results equal the serial order bit for bit."""
    w = _case("bf16", "fwd", T=128 * 19 + 77, H=2, dk=128, dv=128, state_std=0.05, seed=39)
    x = synth.generate(w)
    o_ser, s_ser = run_gpu(x, "fwd", chunk=128, serial=True)
    o_con, s_con = run_gpu(x, "fwd", chunk=128)
    assert np.array_equal(o_ser, o_con) and np.array_equal(s_ser, s_con)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd")
    check(o_con, ref, TOL["bf16"], "out concurrent C=128")
    check(s_con, ref_s, TOL["bf16"], "state concurrent C=128")


def test_chunk128_deterministic():
    """Bitwise the same result over repeated calls."""
    w = _case("bf16", "bi", T=333, H=3, dk=128, dv=128, state_std=0.05, seed=40)
    x = synth.generate(w)
    o1, s1 = run_gpu(x, "bi", chunk=128)
    o2, s2 = run_gpu(x, "bi", chunk=128)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("name", ["bidir480", "causal720"])
def test_chunk128_full_size_sampled_heads(name):
    """The 480p bidirectional (B2 H16 T32760) and 720p causal (B1 H16 T75600,
    nonzero initial state) workloads at 128-token chunks: the GPU computes
    every head, the oracle a sample of (batch, head) chains in full."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.WORKLOADS[name]
    print(f"\n[{name} C=128] generating {w}", flush=True)
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction, chunk=128)
    torch.cuda.synchronize()
    hs = list(dict.fromkeys([(0, 0), (w.B - 1, w.H - 1)]))
    print(f"[{name} C=128] oracle on heads {hs}", flush=True)
    ref, ref_s = oracle.forward_heads(x, hs, w.direction)
    got = np.stack([out[b, :, h].cpu().numpy() for b, h in hs])
    got_s = np.stack([s_out[:, b, h].cpu().numpy() for b, h in hs], axis=1)
    e_o = check(got, ref, TOL[w.dtype], f"{name} C=128 out")
    e_s = check(got_s, ref_s, TOL[w.dtype], f"{name} C=128 state")
    print(f"[{name} C=128] max|err|/RMS: out {e_o:.3e}  state {e_s:.3e}", flush=True)
    del d, out, s_out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("exclusive", ["none", "both"])
def test_chunk128_readout_epilogue_fp32(exclusive):
    """The readout epilogue on fp32 operands at 128-token chunks, inclusive and
    exclusive readouts: against the oracle's scan followed by the oracle's
    epilogue formula (bf16 operands reject this combination)."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = _case("f32", "bi", T=300, H=2, dk=64, dv=64, state_std=0.05, seed=41)
    x = synth.generate(w)
    e = synth.generate_epilogue(w)
    ref, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", exclusive=exclusive)
    ref_y = oracle.readout_epilogue(ref, e["gate"], e["norm_weight"], 1e-6)
    d = {k: to_torch(v) for k, v in x.items()}
    y, _ = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], "bi", chunk=128,
                       exclusive=exclusive, gate=to_torch(e["gate"]), norm_weight=to_torch(e["norm_weight"]),
                       norm_eps=1e-6)
    torch.cuda.synchronize()
    r = check(y.cpu().numpy(), ref_y, TOL["f32"], f"epilogue C=128 exclusive={exclusive}")
    print(f"\nepilogue fp32 C=128 exclusive={exclusive}: {r:.2e} x RMS", flush=True)
