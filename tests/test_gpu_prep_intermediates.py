"""Per-kernel check of the chunk preparation (the state-independent chunk
quantities it leaves in the workspace), against the independent chunked CPU
reference (oracle/chunked_ref.py) in double precision.

After one bidirectional call the workspace holds, per (batch*head, chunk),
in natural token order (layout documented with the workspace layout of the
kernels; replicated here for reading):
  tri  C x C: strictly lower = forward (I + L)^{-1}, strictly upper = reverse;
  pqk  C x C: decayed q^.k^, forward below, reverse above, self terms on the diagonal;
  sc   [dir][chunk][C] x 4: beta, e^g rk, e^g rq, e^(g_last - g) rk;
  pdg  [dir][chunk][stride]: e^(g_last) and three zeros, then the self-term remainder per
       token (0 for fp32 operands).
The state chain fuses everything that depends on the state (Vnew, chunk
outputs, chunk-entry states); those are covered end to end by the parity tests.
"""
import numpy as np
import pytest

import synth
from gdn_testutil import to_torch
from oracle import as_f32
from oracle import chunked_ref as cr

pytestmark = pytest.mark.gpu


def _align(x, a=256):
    return (x + a - 1) // a * a


def _layout(nbh, nc, dirs, mt, C):
    off = 0
    nch = nbh * nc
    tri = off
    off = _align(off + nch * C * C * mt)
    pqk = off
    off = _align(off + nch * C * C * mt)
    sc = off
    off = _align(off + dirs * nch * C * 16)
    pdg = off
    return tri, pqk, sc, pdg


# every block count of the inverse (one 16-token block per side at C = 16,
# two at C = 32, four at C = 64, eight at C = 128: the 128-token preparation
# kernel) and both head widths of the staged q / k
@pytest.mark.parametrize("C,d", [(64, 64), (32, 64), (64, 128), (32, 128), (128, 64), (128, 128), (16, 64),
                                 (16, 128)])
@pytest.mark.parametrize("dtype,tol", [("f32", 2e-5), ("bf16", 1e-2)])
def test_chunk_preparation_outputs(dtype, tol, C, d):
    import torch

    import gated_delta_rule_scan_amd as gdn

    B, H, T = 1, 2, 150  # the last chunk ragged: 22 tokens of 128, 64 or 32, 6 of 16
    w = synth.Workload("prep", B, H, T, d, d, dtype, "bi", 3.0, 0.02, 61)
    x = synth.generate(w)
    dd = {k: to_torch(v) for k, v in x.items()}
    mt = 4 if dtype == "f32" else 2
    prob = gdn.gdn_problem_t(B=B, T=T, H=H, dk=d, dv=d, chunk=C,
                             dtype=gdn.GDN_DTYPE_F32 if dtype == "f32" else gdn.GDN_DTYPE_BF16)
    ws = torch.zeros(gdn.gdn_workspace_bytes(prob, gdn.GDN_DIR_BIDIRECTIONAL), dtype=torch.uint8, device="cuda")
    gdn.forward(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], dd["state_in"], "bi", chunk=C,
                workspace=ws, serial=True)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    nc = (T + C - 1) // C
    nbh = B * H
    o_tri, o_pqk, o_sc, o_pdg = _layout(nbh, nc, 2, mt, C)
    mdt = np.float32 if mt == 4 else np.uint16

    def mat(off, cid):
        a = raw[off + cid * C * C * mt: off + (cid + 1) * C * C * mt].view(mdt).reshape(C, C)
        return as_f32(a).astype(np.float64)

    pds = (C + 4 + 31) // 32 * 32
    q, k = as_f32(x["q"]).astype(np.float64), as_f32(x["k"]).astype(np.float64)
    v = as_f32(x["v"]).astype(np.float64)
    worst = 0.0
    for bh in range(nbh):
        b, h = bh // H, bh % H
        rk = 1.0 / np.maximum(np.linalg.norm(k[b, :, h], axis=-1), 1e-6)
        rq = 1.0 / np.maximum(np.linalg.norm(q[b, :, h], axis=-1), 1e-6)
        for c in range(nc):
            t0, t1 = c * C, min(T, (c + 1) * C)
            n = t1 - t0
            cid = bh * nc + c
            tri, pqk = mat(o_tri, cid)[:n, :n], mat(o_pqk, cid)[:n, :n]
            for slot, rev in ((0, False), (1, True)):
                idx = np.arange(t0, t1)[::-1] if rev else np.arange(t0, t1)
                la = x["log_alpha"][slot, b, idx, h].astype(np.float64)
                bt = x["beta"][slot, b, idx, h].astype(np.float64)
                _, _, it = cr.chunk_step(np.zeros((d, d)), q[b, idx, h], k[b, idx, h], v[b, idx, h], la, bt)
                Ti, P, g = it["Tinv"], it["P"], it["g"]
                if rev:  # back to natural order: the reverse triangles sit above the diagonal
                    Ti, P, g = Ti[::-1, ::-1], P[::-1, ::-1], g[::-1]
                part = np.triu if rev else np.tril
                for got, want in ((part(tri, 1 if rev else -1), part(Ti, 1 if rev else -1)),
                                  (part(pqk, 1 if rev else -1), part(P, 1 if rev else -1))):
                    err = np.max(np.abs(got - want)) / max(1.0, np.max(np.abs(want)))
                    worst = max(worst, err)
                    assert err <= tol, f"bh {bh} chunk {c} {'rev' if rev else 'fwd'}: {err:.2e}"
                # self terms on the diagonal (plus the stored remainder for bf16 operands)
                rec = raw[o_pdg + ((slot * nbh * nc) + cid) * pds * 4:][:pds * 4].view(np.float32)
                self_t = np.diag(pqk) + rec[4:4 + n]
                want_self = np.sum(q[b, t0:t1, h] * k[b, t0:t1, h], axis=-1) * rq[t0:t1] * rk[t0:t1]
                assert np.max(np.abs(self_t - want_self)) <= 2e-6 * max(1.0, np.max(np.abs(want_self)))
                gl = g[-1] if not rev else g[0]  # the chunk's total log-decay
                assert abs(rec[0] - np.exp(gl)) <= (1e-6 + 1e-7 * abs(gl)) * np.exp(gl) + 1e-37
                assert np.all(rec[1:4] == 0)
                # per-token scales, natural order
                sc = raw[o_sc + ((slot * nbh * nc) + cid) * C * 16:][:C * 16].view(np.float32).reshape(C, 4)[:n]
                eg = np.exp(g)
                want_sc = np.stack([x["beta"][slot, b, t0:t1, h], eg * rk[t0:t1], eg * rq[t0:t1],
                                    np.exp(gl - g) * rk[t0:t1]], axis=1)
                # the kernel sums the chunk's log-gates in double and rounds each
                # sum or difference once to fp32 before the exponential, so each
                # factor carries about |exponent| * 2^-24 of relative error plus a
                # few ulp: 1e-6 + 1e-7 (|g| or |g_last - g|), with an absolute floor
                # at the bottom of fp32's normal range (strong decays take e^g below it)
                arg = np.stack([np.zeros(n), np.abs(g), np.abs(g), np.abs(gl - g)], axis=1)
                bad = np.abs(sc - want_sc) > (1e-6 + 1e-7 * arg) * np.abs(want_sc) + 1e-37
                assert not bad.any(), (f"scales bh {bh} chunk {c} slot {slot}: {np.argwhere(bad)[:3]} "
                                       f"got {sc[bad][:3]} want {want_sc[bad][:3]}")
    print(f"\nprep {dtype} C={C} d={d}: worst triangle error {worst:.2e}")
