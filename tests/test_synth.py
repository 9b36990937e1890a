"""The seeded input generator: determinism and the value distributions the
workloads ask for (it holds none of the scan's arithmetic)."""
import os
import subprocess
import sys

import numpy as np

import synth


def _small(dtype="f32", direction="bi", state_std=0.02):
    return synth.Workload("t", 2, 3, 300, 64, 32, dtype, direction, 3.0, state_std, 7)


def test_deterministic_and_seed_sensitive():
    a = synth.generate(_small())
    b = synth.generate(_small())
    for n in ("q", "k", "v", "log_alpha", "beta", "state_in"):
        np.testing.assert_array_equal(a[n], b[n])
    c = synth.generate(_small().replace(seed=8))
    assert not np.array_equal(a["q"], c["q"])
    # streams are distinct
    assert not np.array_equal(a["q"], a["k"][..., :64])


def test_independent_of_thread_count():
    code = ("import synth,numpy as np;x=synth.generate(synth.Workload('t',1,2,500,64,64,'bf16','bi',3.0,0.0,3));"
            "print(int(np.bitwise_xor.reduce(x['q'].ravel().astype(np.uint64)*np.arange(x['q'].size,dtype=np.uint64))),"
            "float(x['beta'].astype(np.float64).sum()))")
    outs = []
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        outs.append(subprocess.check_output([sys.executable, "-c", code], env=env, cwd=root, text=True))
    assert outs[0] == outs[1]


def test_distributions():
    x = synth.generate(synth.Workload("t", 1, 4, 4000, 128, 128, "f32", "bi", 3.0, 0.02, 11))
    nq = np.linalg.norm(x["q"].astype(np.float64), axis=-1)
    np.testing.assert_allclose(nq, 1.0, atol=1e-6)
    v = x["v"].astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    b = x["beta"].astype(np.float64)
    assert b.min() > 0 and b.max() < 1 and abs(b.mean() - 0.5) < 0.01
    la = x["log_alpha"].astype(np.float64)
    # E[-softplus(Z + 3)], Z ~ N(0,1), by quadrature
    z = np.linspace(-9, 9, 20001)
    pdf = np.exp(-z * z / 2) / np.sqrt(2 * np.pi)
    want = -np.trapezoid(np.logaddexp(0, z + 3) * pdf, z)
    assert la.max() < 0 and abs(la.mean() - want) < 0.02
    s = x["state_in"].astype(np.float64)
    assert abs(s.std() - 0.02) < 0.001


def test_bf16_is_nearest_even_of_the_sample():
    f = synth.generate(_small("f32"))
    h = synth.generate(_small("bf16"))
    for n in ("q", "k", "v"):
        x32 = f[n].astype(np.float32)
        u = x32.view(np.uint32).astype(np.uint64)
        rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
        diff = rne != h[n]
        # the only possible disagreements are double-rounding ties through fp32
        assert diff.mean() < 1e-4
        assert np.all(np.abs(rne[diff].astype(np.int32) - h[n][diff].astype(np.int32)) <= 1)
        back = synth.bf16_to_f32(h[n])
        assert np.all(np.abs(back - x32) <= np.abs(x32) * 2.0 ** -8 + 1e-30)


def test_raw_rows_span_scales_and_the_clamp():
    """qk="raw": rows are not unit length; norms span about 1e-3 sqrt(d) to
    1e3 sqrt(d), and every 37th row (global index 5 mod 37) has a norm on
    either side of 1e-6; v and the gates are those of the unit recipe."""
    w = synth.Workload("t", 1, 3, 500, 128, 64, "f32", "bi", 3.0, 0.0, 9, qk="raw")
    x = synth.generate(w)
    u = synth.generate(w.replace(qk="unit"))
    for n in ("v", "log_alpha", "beta"):
        np.testing.assert_array_equal(x[n], u[n])
    for t in ("q", "k"):
        nrm = np.linalg.norm(x[t].astype(np.float64), axis=-1).ravel()
        rows = np.arange(nrm.size)
        tiny = rows % 37 == 5
        assert np.all((nrm[tiny] > 0.45e-6) & (nrm[tiny] < 2.1e-6))
        assert np.any(nrm[tiny] < 1e-6) and np.any(nrm[tiny] > 1e-6)
        big = nrm[~tiny] / np.sqrt(128)
        assert big.min() < 1e-2 and big.max() > 1e2 and big.min() > 1e-4 and big.max() < 1e4
        # direction of each row is that of a N(0, I) draw: not unit length, not constant
        assert not np.allclose(nrm[~tiny], 1.0)
    xb = synth.generate(w.replace(dtype="bf16"))
    np.testing.assert_allclose(synth.bf16_to_f32(xb["q"]), x["q"], rtol=2 ** -8, atol=0)
