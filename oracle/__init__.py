"""Double-precision oracle for the gated delta-rule scan.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this package; the GPU library never does, and the
library shares no code with it.

``forward`` wraps the plain C token-by-token recurrence in ``gdn_oracle.c``
(double precision; see that file for the definition it follows).
``chunked_ref`` holds a second, independent CPU form: the exact chunked
rewriting of the same recurrence, used to pin the oracle and to inspect the
per-chunk quantities (triangular inverse, pseudo-values) the kernels build.

Where each function stands relative to its pins (see ``tests/test_oracle_pins.py``):
every function here is pinned; the inclusive reverse scan is a reading of the
pages (the reverse readout includes the current token), not something the pages
fix, so that single choice is "parity unpinned".  The exclusive readouts (either
direction reading before the token's own write) are pinned by brute force and
by perturbation; where the decay a_t stands in them is a reading.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_SO = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

DIRECTIONS = {"fwd": 0, "rev": 1, "bi": 2}
# which directions read their memory before the token's own write
EXCLUSIVE = {"none": 0, "fwd": 1, "rev": 2, "both": 3}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain IEEE double; no fast-math)."""
    global _lib
    os.makedirs(os.path.dirname(_SO), exist_ok=True)
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                               "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
        _lib = None
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.gdn_oracle_forward.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, p, p, p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.gdn_oracle_forward.restype = ctypes.c_int
        _lib = lib
    return _lib


def as_f32(x: np.ndarray) -> np.ndarray:
    """Exact float32 view of an input: bf16 bit patterns (uint16) are widened."""
    if x.dtype == np.uint16:
        return (np.ascontiguousarray(x).astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


def readout_epilogue(out, gate, norm_weight, norm_eps: float = 1e-6) -> np.ndarray:
    """The readout epilogue ("Video DeltaNet", "Key Contributions" item 1:
    the linear branch's readout is RMS-normalised and passed through a
    sigmoid gate), on every row of ``out`` [..., dv]:

        y = norm_weight * o / sqrt(mean_dv(o^2) + norm_eps) * sigmoid(gate)

    Readings (the page names the normalisation and the gate only): the mean
    runs over the dv channels of one (token, head) row; eps sits inside the
    root; ``norm_weight`` is one vector of dv weights shared by the heads;
    ``gate`` has the shape of ``out`` (bf16 bit patterns or float32)."""
    o = np.asarray(out, np.float64)
    z = as_f32(gate).astype(np.float64)
    w = np.asarray(norm_weight, np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + norm_eps)
    return w * (o / rms) / (1.0 + np.exp(-z))


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(q, k, v, log_alpha, beta, state_in=None, direction: str = "fwd", erase: bool = True,
            nthreads: Optional[int] = None, want_state: bool = True,
            exclusive: str = "none") -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Run the token-by-token recurrence in double precision.

    q, k: [B,T,H,dk]; v: [B,T,H,dv] (float32, or uint16 bf16 bit patterns);
    log_alpha, beta: [dirs,B,T,H]; state_in: [dirs,B,H,dv,dk] or None.
    exclusive: "none", "fwd", "rev" or "both" -- the directions whose readout
    is taken after the decay and before the token's own write (o_t = a_t
    S_{t-1} q^_t), which makes the two scans of a bidirectional call cover
    disjoint regions (see gdn_oracle.c).
    Returns (out [B,T,H,dv] float64, state_out [dirs,B,H,dv,dk] float64 or None).
    """
    q, k, v = as_f32(q), as_f32(k), as_f32(v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dirs = 2 if direction == "bi" else 1
    la = np.ascontiguousarray(log_alpha, dtype=np.float32).reshape(dirs, B, T, H)
    bt = np.ascontiguousarray(beta, dtype=np.float32).reshape(dirs, B, T, H)
    s_in = None if state_in is None else np.ascontiguousarray(state_in, dtype=np.float32).reshape(dirs, B, H, dv, dk)
    out = np.zeros((B, T, H, dv), dtype=np.float64)
    s_out = np.zeros((dirs, B, H, dv, dk), dtype=np.float64) if want_state else None
    nth = nthreads or default_threads()
    nth = max(1, min(nth, B * H * dirs))
    rc = _load().gdn_oracle_forward(
        B, T, H, dk, dv, q.ctypes.data, k.ctypes.data, v.ctypes.data, la.ctypes.data, bt.ctypes.data,
        None if s_in is None else s_in.ctypes.data, None if s_out is None else s_out.ctypes.data,
        out.ctypes.data, DIRECTIONS[direction], int(bool(erase)), EXCLUSIVE[exclusive], nth)
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out, s_out


def forward_heads(inputs: dict, heads, direction: str, nthreads: Optional[int] = None, exclusive: str = "none",
                  erase: bool = True):
    """Oracle on a subset of (batch, head) chains of a full-size input set.

    ``heads`` is a list of (b, h) pairs.  Chains are independent, so this is
    exactly the oracle restricted to those heads.  Returns (out [n,T,dv],
    state_out [dirs,n,dv,dk]) in the order of ``heads``.
    """
    q, k, v = inputs["q"], inputs["k"], inputs["v"]
    la, bt, s_in = inputs["log_alpha"], inputs["beta"], inputs["state_in"]
    # gather each chain as its own batch entry with H = 1
    qs = np.stack([q[b, :, h] for b, h in heads])[:, :, None, :]
    ks = np.stack([k[b, :, h] for b, h in heads])[:, :, None, :]
    vs = np.stack([v[b, :, h] for b, h in heads])[:, :, None, :]
    las = np.stack([la[:, b, :, h] for b, h in heads], axis=1)[..., None]
    bts = np.stack([bt[:, b, :, h] for b, h in heads], axis=1)[..., None]
    ss = None if s_in is None else np.stack([s_in[:, b, h] for b, h in heads], axis=1)[:, :, None]
    out, s_out = forward(qs, ks, vs, las, bts, ss, direction, erase=erase, nthreads=nthreads, exclusive=exclusive)
    return out[:, :, 0, :], (None if s_out is None else s_out[:, :, 0])
