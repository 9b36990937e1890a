"""GPU parity: libgdn (HIP, gfx950) against the double-precision oracle.

Every comparison is element by element over the whole output and the final
state(s), at the tolerance stated in tests/gdn_testutil.py (bf16 inputs:
2e-2 x RMS; fp32 inputs: 1e-4 x RMS).  Sizes span several chunks and a ragged
tail; the oracle finishes each in well under a second.
"""
import numpy as np
import pytest

import oracle
import synth
from gdn_testutil import TOL, check, rel_err, run_gpu

pytestmark = pytest.mark.gpu


def _case(dtype, direction, T, B=1, H=2, dk=64, dv=64, la_shift=3.0, state_std=0.0, seed=0, qk="unit"):
    return synth.Workload("t", B, H, T, dk, dv, dtype, direction, la_shift, state_std, seed, qk=qk)


def _compare(w, chunk=0, dv_tile=0, tol=None):
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], w.direction)
    out, s = run_gpu(x, w.direction, chunk=chunk, dv_tile=dv_tile)
    tol = tol or TOL[w.dtype]
    e1 = check(out, ref, tol, f"out {w}")
    e2 = check(s, ref_s, tol, f"state {w}")
    print(f"\n{w.dtype} {w.direction} T={w.T} d={w.dk}/{w.dv} C={chunk} tile={dv_tile}: out {e1:.2e} state {e2:.2e}",
          flush=True)
    return e1, e2


def test_tiny_causal_fp32():
    """Tiny causal workload: B1 H2 T256 d64 fp32, zero initial state, seed 0."""
    _compare(synth.WORKLOADS["tiny"])


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_directions_ragged(direction, dtype):
    _compare(_case(dtype, direction, T=203, H=3, state_std=0.05, seed=5))


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_raw_qk_normalisation(dtype, direction, chunk):
    """q and k as given, not of unit length: N(0, 1) rows times per-row
    scales from 1e-3 to 1e3, and every 37th row at a norm between 0.5e-6 and
    2e-6 (both sides of the 1e-6 clamp).  The kernels' own row scales
    rq = 1/max(|q|, 1e-6), rk = 1/max(|k|, 1e-6) must reproduce the oracle's
    normalisation in every product they enter (Y, Z, P, the state update)."""
    w = _case(dtype, direction, T=203, H=3, dk=128, dv=64, state_std=0.05, seed=21, qk="raw")
    _compare(w, chunk=chunk)


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
def test_bf16_chunk32(direction):
    """bf16 operands with 32-token chunks (unit-length q, k)."""
    _compare(_case("bf16", direction, T=203, H=3, dk=128, dv=128, state_std=0.05, seed=22), chunk=32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_head_dims_bf16(d, direction):
    _compare(_case("bf16", direction, T=300, B=2, H=2, dk=d, dv=d, state_std=0.02, seed=6))


@pytest.mark.parametrize("chunk", [32, 64])
@pytest.mark.parametrize("dv_tile", [16, 32])
def test_chunk_and_tile_fp32(chunk, dv_tile):
    _compare(_case("f32", "bi", T=333, H=2, dk=64, dv=64, state_std=0.1, seed=7), chunk=chunk, dv_tile=dv_tile)


@pytest.mark.parametrize("direction", ["fwd", "bi"])
def test_wide_tile_fp32_d128(direction):
    """fp32 operands, d = 128, 64-token chunks and 32-wide value tiles."""
    _compare(_case("f32", direction, T=260, H=2, dk=128, dv=128, state_std=0.05, seed=8), dv_tile=32)


@pytest.mark.parametrize("dv_tile", [16, 32])
def test_tile_width_does_not_change_results(dv_tile):
    """The value-tile width changes only the schedule: results are bitwise equal."""
    w = _case("bf16", "bi", T=300, B=2, H=2, dk=128, dv=128, state_std=0.02, seed=12)
    x = synth.generate(w)
    o1, s1 = run_gpu(x, "bi", dv_tile=16)
    o2, s2 = run_gpu(x, "bi", dv_tile=dv_tile)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_concurrent_preparation_matches_serial(direction, dtype):
    """131 chunks on 32 chain workgroups: single-direction scans run the
    preparation pass beside the state chain (the chain waits on per-chunk
    ready flags, and the bf16 chain prefetches a chunk's prepared tiles once
    its flag reads ready); bidirectional bf16 scans run serially.  The
    results are bitwise those of the serial order, and within tolerance of
    the oracle."""
    w = _case(dtype, direction, T=64 * 130 + 17, H=4, dk=64, dv=64, state_std=0.05, seed=13)
    x = synth.generate(w)
    o_ser, s_ser = run_gpu(x, direction, serial=True)
    o_con, s_con = run_gpu(x, direction)
    assert np.array_equal(o_ser, o_con) and np.array_equal(s_ser, s_con)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction)
    check(o_con, ref, TOL[dtype], f"out {w}")
    check(s_con, ref_s, TOL[dtype], f"state {w}")


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_erase_free_variant(direction, dtype):
    """GDN_OPT_NO_ERASE: S_t = a_t S_{t-1} + beta_t v_t k^_t^T (gated linear
    attention), against the oracle's erase-off mode, which is pinned to
    brute-force gated linear attention."""
    w = _case(dtype, direction, T=333, H=3, dk=64, dv=128, state_std=0.05, seed=14)
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction,
                                erase=False)
    out, s = run_gpu(x, direction, erase=False)
    e1 = check(out, ref, TOL[dtype], f"out {w} erase-free")
    e2 = check(s, ref_s, TOL[dtype], f"state {w} erase-free")
    print(f"\nerase-free {dtype} {direction}: out {e1:.2e} state {e2:.2e}", flush=True)


def test_erase_free_variant_concurrent_matches_serial():
    """The erase-free variant on the concurrent preparation path (131 chunks)."""
    w = _case("bf16", "fwd", T=64 * 130 + 5, H=4, dk=128, dv=128, state_std=0.05, seed=15)
    x = synth.generate(w)
    o1, s1 = run_gpu(x, "fwd", serial=True, erase=False)
    o2, s2 = run_gpu(x, "fwd", erase=False)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "fwd", erase=False)
    check(o2, ref, TOL["bf16"], "out erase-free concurrent")


@pytest.mark.parametrize("direction,exclusive", [("fwd", "fwd"), ("rev", "rev"), ("bi", "both"), ("bi", "rev"),
                                                 ("bi", "fwd")])
@pytest.mark.parametrize("dtype,chunk,la_shift", [("f32", 32, 3.0), ("f32", 64, 3.0), ("bf16", 64, 3.0),
                                                   ("f32", 64, -2.0), ("bf16", 64, -2.0)])
def test_exclusive_readout(direction, exclusive, dtype, chunk, la_shift):
    """GDN_OPT_EXCLUSIVE_*: the chosen directions read before the token's own
    write (disjoint regions), against the oracle's exclusive mode, to the
    usual bar on the exclusive output's own RMS; final states are those of
    the inclusive scan, bit for bit.

    With the fast decay (la_shift 3) the token's own write is most of each
    inclusive output, so the exclusive output is about ten times smaller than
    the inclusive one: bf16 scans then add the low parts of the decayed q.k
    tile, and the chunk-local log-gate sums (hundreds within a chunk) are
    taken in double, each decay rounded once."""
    w = _case(dtype, direction, T=203, H=3, dk=64, dv=64, la_shift=la_shift, state_std=0.05, seed=16)
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction,
                                exclusive=exclusive)
    ref_incl, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction)
    out, s = run_gpu(x, direction, chunk=chunk, exclusive=exclusive)
    e1 = check(out, ref, TOL[dtype], f"out {w} exclusive={exclusive}")
    e2 = check(s, ref_s, TOL[dtype], f"state {w} exclusive={exclusive}")
    _, s_incl = run_gpu(x, direction, chunk=chunk)
    assert np.array_equal(s, s_incl)
    print(f"\nexclusive={exclusive} {dtype} {direction} C={chunk} la_shift={la_shift}: out {e1:.2e} x own RMS "
          f"{np.sqrt(np.mean(ref ** 2)):.2e} (inclusive RMS {np.sqrt(np.mean(ref_incl ** 2)):.2e}) state {e2:.2e}",
          flush=True)


@pytest.mark.parametrize("exclusive", ["both", "rev"])
def test_exclusive_readout_erase_free_d128(exclusive):
    """Exclusive readouts with the erase-free variant (brute-force pinned in the oracle), d = 128."""
    w = _case("bf16", "bi", T=300, B=2, H=2, dk=128, dv=128, state_std=0.02, seed=17)
    x = synth.generate(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi",
                                erase=False, exclusive=exclusive)
    out, s = run_gpu(x, "bi", erase=False, exclusive=exclusive)
    check(out, ref, TOL["bf16"], f"out {w} erase-free exclusive={exclusive}")
    check(s, ref_s, TOL["bf16"], f"state {w} erase-free exclusive={exclusive}")


def test_exclusive_readout_concurrent_matches_serial():
    """131 chunks, the reverse scan reading before each token's own write, on
    the concurrent preparation path: equal to the serial order bit for bit."""
    w = _case("bf16", "rev", T=64 * 130 + 17, H=4, dk=64, dv=64, state_std=0.05, seed=18)
    x = synth.generate(w)
    o_ser, s_ser = run_gpu(x, "rev", serial=True, exclusive="rev")
    o_con, s_con = run_gpu(x, "rev", exclusive="rev")
    assert np.array_equal(o_ser, o_con) and np.array_equal(s_ser, s_con)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "rev",
                                exclusive="rev")
    check(o_con, ref, TOL["bf16"], f"out {w} exclusive concurrent")
    check(s_con, ref_s, TOL["bf16"], f"state {w} exclusive concurrent")


def test_calls_from_two_host_threads():
    """Two host threads, each on its own stream with its own buffers, call the
    scan at the same time (bidirectional, serial, and causal on the concurrent
    preparation path, which shares the library stream and events); every
    result equals the same call made alone, bit for bit."""
    import threading

    import torch

    import gated_delta_rule_scan_amd as gdn
    from gdn_testutil import to_torch

    cases = [_case("bf16", "bi", T=64 * 30 + 7, H=4, dk=128, dv=128, state_std=0.05, seed=19),
             _case("bf16", "fwd", T=64 * 130 + 3, H=3, dk=64, dv=64, state_std=0.05, seed=20)]
    inputs = [{k: to_torch(v) for k, v in synth.generate(w).items()} for w in cases]

    def call(d, w, stream=None):
        with torch.cuda.stream(stream or torch.cuda.current_stream()):
            o, s = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], w.direction)
        return o, s

    alone = []
    for d, w in zip(inputs, cases):
        o, s = call(d, w)
        torch.cuda.synchronize()
        alone.append((o.cpu().numpy(), s.cpu().numpy()))
    results = [[None] * 8 for _ in cases]
    errors = []

    def worker(i):
        try:
            st = torch.cuda.Stream()
            for r in range(8):
                o, s = call(inputs[i], cases[i], st)
                results[i][r] = (o, s, st)
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(cases)):
        for o, s, _ in results[i]:
            assert np.array_equal(o.cpu().numpy(), alone[i][0]) and np.array_equal(s.cpu().numpy(), alone[i][1])


@pytest.mark.parametrize("direction,exclusive", [("fwd", "none"), ("rev", "none"), ("bi", "none"), ("bi", "both"),
                                                 ("fwd", "fwd")])
@pytest.mark.parametrize("dtype,dv", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_readout_epilogue(direction, exclusive, dtype, dv):
    """The token scan's readout epilogue (gate and norm weights given):
    against the oracle's scan followed by the oracle's epilogue formula,
    y = w * o / sqrt(mean_dv(o^2) + eps) * sigmoid(gate) per (token, head),
    for inclusive and exclusive readouts; the final states are those of the
    same call without the epilogue, bit for bit."""
    import torch

    import gated_delta_rule_scan_amd as gdn
    from gdn_testutil import to_torch

    w = _case(dtype, direction, T=203, H=3, dk=64, dv=dv, state_std=0.05, seed=19)
    x = synth.generate(w)
    e = synth.generate_epilogue(w)
    ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], direction,
                                exclusive=exclusive)
    ref_y = oracle.readout_epilogue(ref, e["gate"], e["norm_weight"], 1e-6)
    d = {k: to_torch(v) for k, v in x.items()}
    y, s = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], direction,
                       exclusive=exclusive, gate=to_torch(e["gate"]), norm_weight=to_torch(e["norm_weight"]),
                       norm_eps=1e-6)
    o2, s2 = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], direction,
                         exclusive=exclusive)
    torch.cuda.synchronize()
    r = check(y.cpu().numpy(), ref_y, TOL[dtype], f"epilogue {w} exclusive={exclusive}")
    assert torch.equal(s, s2)
    print(f"\nepilogue {dtype} dv={dv} {direction} exclusive={exclusive}: {r:.2e} x RMS", flush=True)


def test_readout_epilogue_eps_and_zero_rows():
    """Rows whose readout is exactly zero (zero v and no initial state on
    some heads: nothing is ever written) stay zero under the epilogue with
    eps > 0, and a large eps dominates the root: against the oracle."""
    import torch

    import gated_delta_rule_scan_amd as gdn
    from gdn_testutil import to_torch

    w = _case("bf16", "bi", T=150, H=3, dk=64, dv=64, seed=20)
    x = synth.generate(w)
    x["v"] = x["v"].copy()
    x["v"][:, :, 1, :] = 0  # head 1 reads zeros everywhere
    e = synth.generate_epilogue(w)
    d = {k: to_torch(v) for k, v in x.items()}
    ref, _ = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi")
    for eps in (1e-6, 0.5):
        y, _ = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], "bi",
                           gate=to_torch(e["gate"]), norm_weight=to_torch(e["norm_weight"]), norm_eps=eps)
        torch.cuda.synchronize()
        yn = y.cpu().numpy()
        assert np.all(yn[:, :, 1, :] == 0)
        check(yn, oracle.readout_epilogue(ref, e["gate"], e["norm_weight"], eps), TOL["bf16"], f"eps={eps}")
