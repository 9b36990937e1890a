"""Seeded synthetic inputs for the gated delta-rule scan workloads.

This module draws random numbers and shapes their distributions; it contains
none of the scan's arithmetic.  Both the double-precision oracle (``oracle/``)
and the GPU library's tests and benchmark take their inputs from here, so the
two sides always see bit-identical operands.

Workload recipes (shapes and value distributions) follow the video-latent
shapes the pages discuss: Wan-style 480p latents of 21 frames x 30x52 tokens
(SANA-Video 2.0 review, "Results": 480p/81 frames) and 720p latents of
45x80 tokens per frame.  Per element:

* q, k ~ N(0, 1), then scaled to unit L2 norm per (batch, token, head) in
  double precision, then rounded to the input dtype (bf16: nearest-even);
  a workload with ``qk="raw"`` instead leaves the rows un-normalised, scales
  each by 10^(6u - 3), u ~ U(0, 1), and puts every 37th row at an L2 norm
  between about 0.5e-6 and 2e-6 (the two sides of a 1e-6 norm clamp), so
  that the consumer's own normalisation is exercised;
* v ~ N(0, 1);
* beta = sigmoid(N(0, 1));
* log_alpha = -softplus(N(0, 1) + shift), shift = 3 (5 for the 720p causal
  rollout; -5 for the slow-decay stress variant);
* state_in ~ N(0, 0.02^2) where a workload asks for a nonzero initial state.

The generator is SplitMix64 used counter-style with Box-Muller normals (see
``synth.c``), so any element can be regenerated independently of thread
count, library version or order.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "_build", "libsynth.so")
_lib = None

# stream identifiers (one independent random stream per tensor)
STREAM_Q, STREAM_K, STREAM_V = 1, 2, 3
STREAM_BETA, STREAM_LOG_ALPHA, STREAM_STATE = 10, 20, 30
STREAM_FRAME_LOG_ALPHA = 40
STREAM_GATE, STREAM_NORM_WEIGHT = 50, 60
STREAM_Q_SCALE, STREAM_K_SCALE = 70, 71


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``_build/libsynth.so`` with gcc (host code only)."""
    global _lib
    os.makedirs(os.path.dirname(_SO), exist_ok=True)
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
        _lib = None
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        i64, u64 = ctypes.c_int64, ctypes.c_uint64
        lib.synth_vectors.argtypes = [u64, u64, i64, i64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, i64]
        lib.synth_vectors.restype = None
        lib.synth_vectors_raw.argtypes = [u64, u64, u64, i64, i64, ctypes.c_int, ctypes.c_void_p, i64]
        lib.synth_vectors_raw.restype = None
        lib.synth_scalars.argtypes = [u64, u64, i64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, i64]
        lib.synth_scalars.restype = None
        lib.synth_bf16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64]
        lib.synth_bf16_to_f32.restype = None
        _lib = lib
    return _lib


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, direction and gate recipe."""

    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str  # "f32" or "bf16" (dtype of q, k, v; gates and state are fp32)
    direction: str  # "fwd", "rev" or "bi"
    la_shift: float = 3.0
    state_std: float = 0.0
    seed: int = 0
    frame: Optional[int] = None  # tokens per streaming call (None: one call)
    qk: str = "unit"  # "unit": q, k rows of unit length; "raw": un-normalised rows (see the module notes)

    @property
    def dirs(self) -> int:
        return 2 if self.direction == "bi" else 1

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # tiny causal case the oracle finishes instantly
    "tiny": Workload("tiny causal fp32 B1 H2 T256 d64", 1, 2, 256, 64, 64, "f32", "fwd", 3.0, 0.0, 0),
    # streaming causal rollout: 21 latent frames of 30x52 tokens, one call per frame
    "stream480": Workload("streaming causal 480p, 21 frames x 1560 tokens, B1 H12 d128", 1, 12, 32760, 128, 128,
                          "bf16", "fwd", 3.0, 0.0, 1, frame=1560),
    # 480p bidirectional DiT linear block (headline workload)
    "bidir480": Workload("480p bidirectional B2 H16 T32760 d128", 2, 16, 32760, 128, 128, "bf16", "bi", 3.0, 0.0, 2),
    # 720p long causal rollout with a nonzero initial state
    "causal720": Workload("720p causal B1 H16 T75600 d128", 1, 16, 75600, 128, 128, "bf16", "fwd", 5.0, 0.02, 3),
    # 720p long-duration bidirectional: 31 frames x 3600 tokens
    "bidir720": Workload("720p long bidirectional B1 H24 T111600 d128", 1, 24, 111600, 128, 128, "bf16", "bi", 3.0, 0.0, 4),
    # slow-decay stress variant of the 720p causal rollout (mean decay ~0.99 per token)
    "causal720_slow": Workload("720p causal slow decay B1 H16 T75600 d128", 1, 16, 75600, 128, 128, "bf16", "fwd",
                               -5.0, 0.02, 5),
}


def _vectors(seed, stream, rows, d, unit, dtype):
    if d > 1024:
        raise ValueError("head dimension above 1024 is not supported by the generator")
    lib = _load()
    if dtype == "bf16":
        out = np.empty((rows, d), dtype=np.uint16)
        lib.synth_vectors(seed, stream, rows, d, int(unit), 1, out.ctypes.data, 0)
    else:
        out = np.empty((rows, d), dtype=np.float32)
        lib.synth_vectors(seed, stream, rows, d, int(unit), 0, out.ctypes.data, 0)
    return out


def _vectors_raw(seed, stream, scale_stream, rows, d, dtype):
    if d > 1024:
        raise ValueError("head dimension above 1024 is not supported by the generator")
    lib = _load()
    if dtype == "bf16":
        out = np.empty((rows, d), dtype=np.uint16)
        lib.synth_vectors_raw(seed, stream, scale_stream, rows, d, 1, out.ctypes.data, 0)
    else:
        out = np.empty((rows, d), dtype=np.float32)
        lib.synth_vectors_raw(seed, stream, scale_stream, rows, d, 0, out.ctypes.data, 0)
    return out


def _scalars(seed, stream, n, kind, p0):
    lib = _load()
    out = np.empty(n, dtype=np.float32)
    lib.synth_scalars(seed, stream, n, kind, float(p0), out.ctypes.data, 0)
    return out


def generate(w: Workload, T: Optional[int] = None) -> dict:
    """Draw all inputs of workload ``w`` (optionally with a different length T).

    Returns numpy arrays: q, k [B,T,H,dk] and v [B,T,H,dv] as uint16 bf16 bit
    patterns (dtype "bf16") or float32; log_alpha, beta [dirs,B,T,H] float32;
    state_in [dirs,B,H,dv,dk] float32 or None.
    """
    T = w.T if T is None else T
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    rows = B * T * H
    if w.qk == "raw":
        q = _vectors_raw(w.seed, STREAM_Q, STREAM_Q_SCALE, rows, dk, w.dtype).reshape(B, T, H, dk)
        k = _vectors_raw(w.seed, STREAM_K, STREAM_K_SCALE, rows, dk, w.dtype).reshape(B, T, H, dk)
    elif w.qk == "unit":
        q = _vectors(w.seed, STREAM_Q, rows, dk, True, w.dtype).reshape(B, T, H, dk)
        k = _vectors(w.seed, STREAM_K, rows, dk, True, w.dtype).reshape(B, T, H, dk)
    else:
        raise ValueError(f"qk must be 'unit' or 'raw', not {w.qk!r}")
    v = _vectors(w.seed, STREAM_V, rows, dv, False, w.dtype).reshape(B, T, H, dv)
    la = np.stack([_scalars(w.seed, STREAM_LOG_ALPHA + d, rows, 2, w.la_shift) for d in range(w.dirs)])
    beta = np.stack([_scalars(w.seed, STREAM_BETA + d, rows, 1, 0.0) for d in range(w.dirs)])
    la = la.reshape(w.dirs, B, T, H)
    beta = beta.reshape(w.dirs, B, T, H)
    state_in = None
    if w.state_std > 0:
        n = B * H * dv * dk
        state_in = np.stack([_scalars(w.seed, STREAM_STATE + d, n, 0, w.state_std) for d in range(w.dirs)])
        state_in = state_in.reshape(w.dirs, B, H, dv, dk)
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, state_in=state_in)


def generate_frames(w: Workload, frame: int, T: Optional[int] = None) -> dict:
    """Inputs of the frame-wise operator for workload ``w`` with ``frame``
    tokens per frame: as ``generate`` (per-token beta), but one log-decay per
    frame, log_alpha [dirs,B,NF,H], drawn with the workload's recipe."""
    x = generate(w, T)
    T = x["q"].shape[1]
    NF = (T + frame - 1) // frame
    n = w.B * NF * w.H
    la = np.stack([_scalars(w.seed, STREAM_FRAME_LOG_ALPHA + d, n, 2, w.la_shift) for d in range(w.dirs)])
    x["log_alpha"] = la.reshape(w.dirs, w.B, NF, w.H)
    return x


def generate_epilogue(w: Workload, T: Optional[int] = None) -> dict:
    """Inputs of the readout epilogue: gate logits [B,T,H,dv] ~ N(0, 1) in the
    workload's dtype (bf16 bit patterns or float32) and one vector of norm
    weights [dv] ~ 1 + N(0, 0.1^2), float32."""
    T = w.T if T is None else T
    z = _vectors(w.seed, STREAM_GATE, w.B * T * w.H, w.dv, False, w.dtype).reshape(w.B, T, w.H, w.dv)
    nw = 1.0 + _scalars(w.seed, STREAM_NORM_WEIGHT, w.dv, 0, 0.1)
    return dict(gate=z, norm_weight=nw.astype(np.float32))


def normals(seed: int, stream: int, shape, std: float = 1.0) -> np.ndarray:
    """Plain N(0, std^2) float32 array from a named stream (for tests)."""
    n = int(np.prod(shape))
    return _scalars(seed, stream, n, 0, std).reshape(shape)


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    if x.dtype == np.float32:
        return x
    if x.dtype != np.uint16:
        raise TypeError("expected uint16 bf16 bit patterns or float32")
    x = np.ascontiguousarray(x)
    out = np.empty(x.shape, dtype=np.float32)
    _load().synth_bf16_to_f32(x.ctypes.data, out.ctypes.data, x.size)
    return out
