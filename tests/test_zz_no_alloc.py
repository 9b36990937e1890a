"""gdn_forward_noalloc on the GPU: the entry point for callers that cannot
allocate (its workspace is the library's fixed device scratch) gives, bit for
bit, the results of gdn_forward with a caller-provided workspace.  Two calls in
a row, the second on a smaller problem, so the second call runs on scratch
that still holds the first call's contents."""
import numpy as np
import pytest

import synth
from gdn_testutil import TOL, check, to_torch

pytestmark = pytest.mark.gpu


def _call(entry, w, x):
    import torch

    import gated_delta_rule_scan_amd as gdn

    d = {k: to_torch(v) for k, v in x.items()}
    dirs = w.dirs
    out = torch.full((w.B, w.T, w.H, w.dv), float("nan"), dtype=torch.float32, device="cuda")
    s_out = torch.full((dirs, w.B, w.H, w.dv, w.dk), float("nan"), dtype=torch.float32, device="cuda")
    dt = gdn.GDN_DTYPE_BF16 if w.dtype == "bf16" else gdn.GDN_DTYPE_F32
    prob = gdn.make_problem(w.B, w.T, w.H, w.dk, w.dv, dt)
    prob.stream = torch.cuda.current_stream().cuda_stream
    keep = []
    if entry == "forward":
        nb = gdn.gdn_workspace_bytes(prob, gdn.DIRECTIONS[w.direction])
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        keep.append(ws)
        prob.workspace, prob.workspace_bytes = ws.data_ptr(), nb
        prob.options = gdn.GDN_OPT_SERIAL
        fn = gdn.gdn_forward
    else:
        fn = gdn.gdn_forward_noalloc
    si = d["state_in"]
    st = fn(prob, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), d["log_alpha"].data_ptr(),
            d["beta"].data_ptr(), None if si is None else si.data_ptr(), s_out.data_ptr(), out.data_ptr(),
            gdn.DIRECTIONS[w.direction])
    assert st == gdn.GDN_OK, gdn.gdn_status_string(st)
    torch.cuda.synchronize()
    return out.cpu().numpy(), s_out.cpu().numpy()


def test_noalloc_equals_forward_on_two_calls_the_second_smaller():
    import oracle

    first = synth.Workload("noalloc 1", 1, 12, 1560, 128, 128, "bf16", "bi", 3.0, 0.02, 41)
    second = synth.Workload("noalloc 2", 1, 4, 333, 64, 128, "bf16", "fwd", 3.0, 0.05, 42)
    for w in (first, second):
        x = synth.generate(w)
        print(f"\n[noalloc] {w}", flush=True)
        o_na, s_na = _call("noalloc", w, x)
        o_fw, s_fw = _call("forward", w, x)
        assert np.array_equal(o_na, o_fw) and np.array_equal(s_na, s_fw)
        ref, ref_s = oracle.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], w.direction)
        e1 = check(o_na, ref, TOL[w.dtype], f"noalloc out {w.name}")
        e2 = check(s_na, ref_s, TOL[w.dtype], f"noalloc state {w.name}")
        print(f"[noalloc] {w.name}: bitwise equal to gdn_forward; out {e1:.2e} state {e2:.2e} x RMS", flush=True)


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    import torch

    import gated_delta_rule_scan_amd as gdn

    prob = gdn.make_problem(2, 32760, 16, 128, 128, gdn.GDN_DTYPE_BF16)
    prob.stream = torch.cuda.current_stream().cuda_stream
    x = torch.zeros(16, device="cuda")
    p = x.data_ptr()
    st = gdn.gdn_forward_noalloc(prob, p, p, p, p, p, None, None, p, gdn.GDN_DIR_BIDIRECTIONAL)
    assert st == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
