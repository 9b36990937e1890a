"""Double-precision oracle for the frame-wise delta operator (Video Delta Attention)
and its two neighbours on the same frame machinery.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the test suite, the
smoke check and the benchmark's CPU-baseline leg may use it; the GPU library
shares no code with it.

Definition ("Video DeltaNet", "Key Contributions" item 2, and "Methodology in
Plain English"): the memory is written once per latent frame, as the minimiser
of a regularised least-squares objective -- squared distance from the decayed
previous memory plus the beta-weighted squared recall errors of the frame's
keys,

    S_t = argmin_S  ||S - Sbar_t||_F^2 + sum_{i in frame t} beta_i ||S k^_i - v_i||^2,
    Sbar_t = a_t S_{t-1},

whose closed form is the one the page gives,

    S_t = (Sbar_t + B_t) (I + A_t)^{-1},
    A_t = sum_i beta_i k^_i k^_i^T  (dk x dk),   B_t = sum_i beta_i v_i k^_i^T  (dv x dk).

The additive frame write the same page contrasts it with ("Main Findings",
last item: SANA-WM's batched per-token updates with 1/sqrt(U) key scaling):
every token's delta-rule correction is computed from the same decayed memory
and the corrections are summed, with keys scaled by 1/sqrt(U), U the frame's
token count,

    S_t = Sbar_t + sum_i beta_i (v_i - Sbar_t k~_i) k~_i^T,   k~_i = k^_i / sqrt(U).

Disjoint-region readout ("Methodology in Plain English": each scan sees its own
non-overlapping part of the video, so adding the readouts counts no frame
twice, and the text's state starts each direction at half weight, S_T/2): with a readout lag
d >= 0, a token of frame t reads the forward state after frame t - d and the
reverse state after frame t + d (the initial state where that frame does not
exist).  d = 0 is the inclusive readout.

Readout epilogue ("Key Contributions" item 1: a sigmoid gate and RMS
normalisation of the linear branch's readout), on the summed readout o of
each (token, head): y = norm_weight * o / sqrt(mean(o^2) + eps) * sigmoid(gate).

Readings taken where the page is silent:
  * q and k are normalised as in the token scan: x^ = x / max(|x|_2, 1e-6);
  * one decay a_t = exp(log_alpha_t) per frame, one write strength beta_i per
    token (beta >= 0 keeps A_t positive semi-definite);
  * every token of frame t reads the state after its own frame's write,
    o_i = S_t q^_i (as the token scan's readout includes the current token),
    unless a readout lag is given;
  * frames are consecutive runs of ``frame`` tokens, the last one possibly
    shorter (its U is its own token count); the reverse scan visits the frames
    last to first; the bidirectional output is the sum of both readouts, each
    direction with its own gates and initial state;
  * the epilogue's mean runs over the dv channels of one head; norm_weight is
    one vector of dv weights shared by the heads.

The solve is a library routine (numpy.linalg.solve on the symmetric system);
everything else is the definition written out.  Pins: tests/test_vda_oracle_pins.py.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import as_f32, readout_epilogue

EPS = 1e-6


def _normalise_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, EPS)


def frame_update(S_prev: np.ndarray, a: float, kh: np.ndarray, v: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """One frame's write: (a S_prev + B) (I + A)^{-1}; kh [n, dk] unit rows, v [n, dv], beta [n]."""
    dk = kh.shape[1]
    A = (kh * beta[:, None]).T @ kh
    Bm = (v * beta[:, None]).T @ kh
    R = a * S_prev + Bm
    # S (I + A) = R  <=>  (I + A) S^T = R^T   (I + A symmetric)
    return np.linalg.solve(np.eye(dk) + A, R.T).T


def frame_update_additive(S_prev: np.ndarray, a: float, kh: np.ndarray, v: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """One additive frame write: per-token delta corrections from the same decayed
    memory, summed, keys scaled by 1/sqrt(U); kh [U, dk] unit rows, v [U, dv], beta [U]."""
    U = kh.shape[0]
    ks = kh / np.sqrt(U)
    Sbar = a * S_prev
    S = Sbar.copy()
    for i in range(U):
        S += beta[i] * np.outer(v[i] - Sbar @ ks[i], ks[i])
    return S


def forward(q, k, v, log_alpha, beta, state_in: Optional[np.ndarray], direction: str, frame: int,
            return_states: bool = False, write: str = "inverse", lag: int = 0, gate=None, norm_weight=None,
            norm_eps: float = 1e-6):
    """q, k [B,T,H,dk], v [B,T,H,dv] (float32 or bf16 bit patterns); log_alpha
    [dirs,B,NF,H] (one per frame); beta [dirs,B,T,H]; state_in [dirs,B,H,dv,dk]
    or None.  ``write``: "inverse" (the frame-wise delta operator) or
    "additive" (summed per-token corrections, keys / sqrt(U)); ``lag``: the
    readout lag in frames; ``gate`` [B,T,H,dv] (float32 or bf16 bit patterns)
    with ``norm_weight`` [dv]: the readout epilogue.  Returns (out [B,T,H,dv],
    state_out [dirs,B,H,dv,dk]) in float64, plus the state after every frame
    [dirs,B,H,NF,dv,dk] if ``return_states``."""
    q = as_f32(q).astype(np.float64)
    k = as_f32(k).astype(np.float64)
    v = as_f32(v).astype(np.float64)
    la = np.asarray(log_alpha, dtype=np.float64)
    bt = np.asarray(beta, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dirs = 2 if direction == "bi" else 1
    NF = (T + frame - 1) // frame
    update = {"inverse": frame_update, "additive": frame_update_additive}[write]
    out = np.zeros((B, T, H, dv))
    s_out = np.zeros((dirs, B, H, dv, dk))
    states = np.zeros((dirs, B, H, NF, dv, dk)) if return_states else None
    qh = _normalise_rows(q)
    kh = _normalise_rows(k)
    for slot in range(dirs):
        rev = direction == "rev" or (direction == "bi" and slot == 1)
        for b in range(B):
            for h in range(H):
                S0 = np.zeros((dv, dk)) if state_in is None else np.asarray(state_in, np.float64)[slot, b, h].copy()
                S = S0
                after = [None] * NF  # the state after each frame's write
                for f in (range(NF - 1, -1, -1) if rev else range(NF)):
                    t0, t1 = f * frame, min(T, (f + 1) * frame)
                    S = update(S, float(np.exp(la[slot, b, f, h])), kh[b, t0:t1, h], v[b, t0:t1, h], bt[slot, b, t0:t1, h])
                    after[f] = S
                    if return_states:
                        states[slot, b, h, f] = S
                for f in range(NF):
                    t0, t1 = f * frame, min(T, (f + 1) * frame)
                    src = f + lag if rev else f - lag
                    R = after[src] if 0 <= src < NF else S0
                    out[b, t0:t1, h] += qh[b, t0:t1, h] @ R.T
                s_out[slot, b, h] = S
    if gate is not None:
        out = readout_epilogue(out, gate, norm_weight, norm_eps)
    if return_states:
        return out, s_out, states
    return out, s_out
