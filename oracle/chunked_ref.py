"""Chunked double-precision form of the gated delta-rule scan (CPU, numpy).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The recurrence S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t
can be evaluated a chunk of n tokens at a time without approximation.  The
pages only name the idea ("chunk-wise bidirectional scans" and a fused blocked
small-matrix inverse, "Video DeltaNet", "Key Contributions" item 4); the
equations below are derived here from the recurrence.

For a chunk entered with state S (processing order r = 0..n-1):

  g_r   = sum_{j<=r} log_alpha_j                   (chunk-local inclusive cumsum)
  G_ri  = exp(g_r - g_i) for i <= r, else 0
  L     = strictly_lower( diag(beta) (K^ K^^T) * G )
  Tinv  = (I + L)^{-1}                             (unit lower triangular)
  X     = diag(beta) (V - diag(e^g) K^ S^T)        (pseudo-values against the entry state)
  Vnew  = Tinv X                                   (the delta-rule update vectors u_r)
  O     = diag(e^g) Q^ S^T + ((Q^ K^^T) * G) Vnew  (G includes the diagonal)
  S'    = e^{g_{n-1}} S + Vnew^T diag(e^{g_{n-1} - g}) K^

Derivation: unrolling the recurrence inside the chunk gives
S_r = e^{g_r} S + sum_{i<=r} G_ri u_i k^_i^T with u_r = beta_r (v_r - a_r S_{r-1} k^_r);
substituting S_{r-1} into u_r yields the unit-lower system (I + L) U = X.

This module is pinned against the token-by-token oracle to ~1e-12 for several
chunk sizes and ragged tails.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def _normalise_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, EPS)


def chunk_indices(T: int, C: int, reverse: bool):
    """Token indices of each chunk in processing order.

    Chunk boundaries are the physical ones [0,C), [C,2C), ... for both
    directions; the reverse scan visits the chunks last-to-first and the
    tokens inside a chunk last-to-first.
    """
    starts = list(range(0, T, C))
    chunks = [np.arange(s, min(s + C, T)) for s in starts]
    if reverse:
        chunks = [c[::-1] for c in chunks[::-1]]
    return chunks


def chunk_step(S, q, k, v, la, beta):
    """One chunk: returns (O, S_next, dict of intermediates). Inputs in processing order."""
    qh, kh = _normalise_rows(q), _normalise_rows(k)
    n = k.shape[0]
    g = np.cumsum(la)
    diff = g[:, None] - g[None, :]
    mask = np.tril(np.ones((n, n), dtype=bool))
    Gam = np.where(mask, np.exp(np.where(mask, diff, 0.0)), 0.0)
    L = np.tril(beta[:, None] * (kh @ kh.T) * Gam, -1)
    Tinv = np.linalg.inv(np.eye(n) + L)
    X = beta[:, None] * (v - np.exp(g)[:, None] * (kh @ S.T))
    Vnew = Tinv @ X
    O = np.exp(g)[:, None] * (qh @ S.T) + ((qh @ kh.T) * Gam) @ Vnew
    S_next = np.exp(g[-1]) * S + Vnew.T @ (np.exp(g[-1] - g)[:, None] * kh)
    return O, S_next, dict(g=g, Tinv=Tinv, X=X, Vnew=Vnew, P=(qh @ kh.T) * Gam)


def chain(q, k, v, la, beta, S0, C: int, reverse: bool = False):
    """One (batch, head) chain.  q,k [T,dk]; v [T,dv]; la, beta [T]; S0 [dv,dk]."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64, copy=True)
    out = np.zeros((T, v.shape[1]))
    for idx in chunk_indices(T, C, reverse):
        O, S, _ = chunk_step(S, q[idx].astype(np.float64), k[idx].astype(np.float64),
                             v[idx].astype(np.float64), la[idx].astype(np.float64),
                             beta[idx].astype(np.float64))
        out[idx] = O
    return out, S


def forward(q, k, v, log_alpha, beta, state_in=None, direction: str = "fwd", C: int = 64):
    """Same interface and layouts as ``oracle.forward`` (float64 out), chunked evaluation."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dirs = 2 if direction == "bi" else 1
    out = np.zeros((B, T, H, dv))
    s_out = np.zeros((dirs, B, H, dv, dk))
    for b in range(B):
        for h in range(H):
            for d in range(dirs):
                reverse = direction == "rev" or (direction == "bi" and d == 1)
                S0 = np.zeros((dv, dk)) if state_in is None else state_in[d, b, h]
                o, S = chain(q[b, :, h], k[b, :, h], v[b, :, h], log_alpha[d, b, :, h], beta[d, b, :, h],
                             S0, C, reverse)
                out[b, :, h] += o
                s_out[d, b, h] = S
    return out, s_out
