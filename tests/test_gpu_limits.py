"""GPU runs at the size limits of include/gdn.h, checked against the oracle.

* B*H = 65535 (the largest batch*head count), a ragged 70-token sequence,
  bidirectional: the oracle recomputes a sample of (batch, head) chains in full.
* The longest sequence whose rows fit 32-bit byte offsets at H = 1, d = 128:
  T = 8,388,543 tokens ((T + 64) * H * d * 4 < 2^32), bidirectional.  The
  oracle cannot run 8.4 million tokens, so the gates reset a direction's
  memory where a window of tokens must not depend on what lies outside it: a
  log-gate of -1000 makes a_t = 0 exactly (in double, and as exp2 in fp32), so
  S_t = beta_t v_t k^_t^T whatever came before.  With a forward reset at the
  first token of a window and a reverse reset at its last token, the outputs
  of the window are those of the oracle run on the window alone (forward
  memory starting empty at the reset, reverse memory likewise).  Three windows
  are checked: the head (forward initial state from the caller, reverse
  memory reset at the window's end), a window in the middle, and the tail
  (reverse initial state from the caller, forward memory reset at its start);
  the head gives the final reverse state and the tail the final forward state.
  The inputs outside the windows repeat one generated block of 2^20 tokens,
  which keeps the distributions and costs seconds instead of a minute.
"""
import numpy as np
import pytest

import oracle
import synth
from gdn_testutil import TOL, check, to_torch

pytestmark = pytest.mark.gpu


def test_largest_batch_head_count():
    import torch

    import gated_delta_rule_scan_amd as gdn

    w = synth.Workload("max B*H", 3, 21845, 70, 64, 64, "bf16", "bi", 3.0, 0.0, 31)
    assert w.B * w.H == 65535
    print(f"\n[max B*H] generating {w}", flush=True)
    x = synth.generate(w)
    d = {k: to_torch(v) for k, v in x.items()}
    out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, "bi")
    torch.cuda.synchronize()
    heads = [(0, 0), (2, 21844), (1, 10922), (2, 0)]
    ref, ref_s = oracle.forward_heads(x, heads, "bi")
    got = np.stack([out[b, :, h].cpu().numpy() for b, h in heads])
    got_s = np.stack([s_out[:, b, h].cpu().numpy() for b, h in heads], axis=1)
    e_o = check(got, ref, TOL["bf16"], "max B*H out")
    e_s = check(got_s, ref_s, TOL["bf16"], "max B*H state")
    print(f"[max B*H] max|err|/RMS: out {e_o:.2e} state {e_s:.2e}", flush=True)


def _tiled(a, axis, n):
    """a repeated along `axis` up to length n (filled in place)."""
    shape = list(a.shape)
    shape[axis] = n
    out = np.empty(shape, a.dtype)
    L = a.shape[axis]
    for i in range(0, n, L):
        k = min(L, n - i)
        dst = [slice(None)] * a.ndim
        src = [slice(None)] * a.ndim
        dst[axis], src[axis] = slice(i, i + k), slice(0, k)
        out[tuple(dst)] = a[tuple(src)]
    return out


def test_longest_sequence_at_one_head():
    import torch

    import gated_delta_rule_scan_amd as gdn

    d_head = 128
    T = (1 << 32) // (d_head * 4) - 64 - 1
    assert (T + 64) * d_head * 4 < (1 << 32) <= (T + 65) * d_head * 4
    assert gdn.workspace_bytes(1, T, 1, d_head, d_head, "bf16", "bi") > 0
    base = synth.generate(synth.Workload("block", 1, 1, 1 << 20, d_head, d_head, "bf16", "bi", 3.0, 0.02, 32))
    print(f"\n[max T] tiling a 2^20-token block to T = {T}", flush=True)
    x = {"q": _tiled(base["q"], 1, T), "k": _tiled(base["k"], 1, T), "v": _tiled(base["v"], 1, T),
         "log_alpha": _tiled(base["log_alpha"], 2, T), "beta": _tiled(base["beta"], 2, T),
         "state_in": base["state_in"]}
    W = 300
    m = T // 2 + 37  # a window in the middle, not aligned to any chunk
    la = x["log_alpha"]
    la[1, 0, W - 1, 0] = -1000.0   # head window: reverse memory starts empty at its last token
    la[0, 0, m, 0] = -1000.0       # middle window: both directions start empty at its ends
    la[1, 0, m + W - 1, 0] = -1000.0
    la[0, 0, T - W, 0] = -1000.0   # tail window: forward memory starts empty at its first token
    d = {k: to_torch(v) for k, v in x.items()}
    print("[max T] GPU run", flush=True)
    out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], "bi")
    torch.cuda.synchronize()
    del d

    zero = np.zeros_like(x["state_in"][:1])

    def window(t0, t1, s_in):
        sl = slice(t0, t1)
        return oracle.forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["log_alpha"][:, :, sl],
                              x["beta"][:, :, sl], s_in, "bi")

    s_in = x["state_in"]
    checks = [("head", 0, W, np.concatenate([s_in[:1], zero])),
              ("middle", m, m + W, None),
              ("tail", T - W, T, np.concatenate([zero, s_in[1:]]))]
    for name, t0, t1, st in checks:
        ref, ref_s = window(t0, t1, st)
        got = out[:, t0:t1].cpu().numpy()
        e = check(got, ref, TOL["bf16"], f"max T {name} window out")
        print(f"[max T] {name} window [{t0}, {t1}): max|err|/RMS {e:.2e}", flush=True)
        if name == "head":
            e = check(s_out[1].cpu().numpy(), ref_s[1], TOL["bf16"], "max T final reverse state")
            print(f"[max T] final reverse state: {e:.2e}", flush=True)
        if name == "tail":
            e = check(s_out[0].cpu().numpy(), ref_s[0], TOL["bf16"], "max T final forward state")
            print(f"[max T] final forward state: {e:.2e}", flush=True)
    del out, s_out
    torch.cuda.empty_cache()


def _vda_heads_oracle(x, heads, frame):
    from oracle import vda as vda_oracle

    refs, ref_ss = [], []
    for b, h in heads:
        sl = lambda a: np.ascontiguousarray(a[b:b + 1, :, h:h + 1])
        gl = lambda a: np.ascontiguousarray(a[:, b:b + 1, :, h:h + 1])
        r, rs = vda_oracle.forward(sl(x["q"]), sl(x["k"]), sl(x["v"]), gl(x["log_alpha"]), gl(x["beta"]), None, "bi",
                                   frame)
        refs.append(r[0, :, 0])
        ref_ss.append(rs[:, 0, 0])
    return np.stack(refs), np.stack(ref_ss, axis=1)


def test_vda_largest_batch_head_count():
    """The frame-wise operator at B*H = 65535: 70 tokens in frames of 40 (a
    ragged second frame), bidirectional, sampled chains against the oracle."""
    import torch

    import gated_delta_rule_scan_amd as gdn

    frame = 40
    w = synth.Workload("vda max B*H", 3, 21845, 70, 64, 64, "bf16", "bi", -3.0, 0.0, 33)
    print(f"\n[vda max B*H] generating {w}", flush=True)
    x = synth.generate_frames(w, frame)
    d = {k: to_torch(v) for k, v in x.items()}
    out, s_out = gdn.vda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], None, "bi", frame)
    torch.cuda.synchronize()
    heads = [(0, 0), (2, 21844), (1, 10922)]
    ref, ref_s = _vda_heads_oracle(x, heads, frame)
    got = np.stack([out[b, :, h].cpu().numpy() for b, h in heads])
    got_s = np.stack([s_out[:, b, h].cpu().numpy() for b, h in heads], axis=1)
    e_o = check(got, ref, TOL["bf16"], "vda max B*H out")
    e_s = check(got_s, ref_s, TOL["bf16"], "vda max B*H state")
    print(f"[vda max B*H] max|err|/RMS: out {e_o:.2e} state {e_s:.2e}", flush=True)
    del d, out, s_out
    torch.cuda.empty_cache()


def test_vda_longest_sequence_at_one_head():
    """The frame-wise operator on the longest sequence at H = 1, d = 128
    (T = 8,388,543 in 5,378 frames of 1,560 tokens, the last one 423 long),
    bidirectional.  A per-frame log-gate of -1000 restarts a direction's
    memory at that frame (S_t = B_t (I + A_t)^-1), so windows of three frames
    are checked against the oracle run on them alone, as for the token scan."""
    import torch

    from oracle import vda as vda_oracle
    import gated_delta_rule_scan_amd as gdn

    d_head, frame = 128, 1560
    T = (1 << 32) // (d_head * 4) - 64 - 1
    NF = -(-T // frame)
    base = synth.generate_frames(synth.Workload("block", 1, 1, 1 << 20, d_head, d_head, "bf16", "bi", -3.0, 0.02, 34),
                                 frame)
    print(f"\n[vda max T] tiling a 2^20-token block to T = {T} ({NF} frames)", flush=True)
    x = {"q": _tiled(base["q"], 1, T), "k": _tiled(base["k"], 1, T), "v": _tiled(base["v"], 1, T),
         "log_alpha": _tiled(base["log_alpha"], 2, NF), "beta": _tiled(base["beta"], 2, T),
         "state_in": base["state_in"]}
    n = 3
    fm = NF // 2 + 5
    la = x["log_alpha"]
    la[1, 0, n - 1, 0] = -1000.0
    la[0, 0, fm, 0] = -1000.0
    la[1, 0, fm + n - 1, 0] = -1000.0
    la[0, 0, NF - n, 0] = -1000.0
    d = {k: to_torch(v) for k, v in x.items()}
    print("[vda max T] GPU run", flush=True)
    out, s_out = gdn.vda_forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["state_in"], "bi", frame)
    torch.cuda.synchronize()
    del d

    zero = np.zeros_like(x["state_in"][:1])
    s_in = x["state_in"]
    for name, f0, f1, st in (("head", 0, n, np.concatenate([s_in[:1], zero])), ("middle", fm, fm + n, None),
                             ("tail", NF - n, NF, np.concatenate([zero, s_in[1:]]))):
        t0, t1 = f0 * frame, min(T, f1 * frame)
        sl = slice(t0, t1)
        ref, ref_s = vda_oracle.forward(x["q"][:, sl], x["k"][:, sl], x["v"][:, sl], x["log_alpha"][:, :, f0:f1],
                                        x["beta"][:, :, sl], st, "bi", frame)
        e = check(out[:, t0:t1].cpu().numpy(), ref, TOL["bf16"], f"vda max T {name} window out")
        print(f"[vda max T] {name} frames [{f0}, {f1}) tokens [{t0}, {t1}): max|err|/RMS {e:.2e}", flush=True)
        if name == "head":
            e = check(s_out[1].cpu().numpy(), ref_s[1], TOL["bf16"], "vda max T final reverse state")
            print(f"[vda max T] final reverse state: {e:.2e}", flush=True)
        if name == "tail":
            e = check(s_out[0].cpu().numpy(), ref_s[0], TOL["bf16"], "vda max T final forward state")
            print(f"[vda max T] final forward state: {e:.2e}", flush=True)
    del out, s_out
    torch.cuda.empty_cache()
