"""Host-side checks of the frame-wise operator's C ABI (gdn_vda_*): the ctypes
mirror of gdn_vda_problem_t matches the C layout, workspace sizing, and every
argument check returns its status before anything is enqueued.  A valid call
on a machine without a GPU reaches the launch and reports GDN_ERR_HIP."""
import os
import subprocess

import pytest

import gated_delta_rule_scan_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BASE = 1 << 40


def _prob(B=1, T=300, H=2, dk=128, dv=128, frame=100, dtype=gdn.GDN_DTYPE_BF16, ws=0, wsb=0):
    return gdn.gdn_vda_problem_t(B=B, T=T, H=H, dk=dk, dv=dv, frame=frame, dtype=dtype, workspace=ws or None,
                                 workspace_bytes=wsb)


def _bufs(B=1, T=300, H=2, dk=128, dv=128, frame=100, es=2, dirs=1):
    NF = (T + frame - 1) // frame
    sizes = dict(q=B * T * H * dk * es, k=B * T * H * dk * es, v=B * T * H * dv * es, la=dirs * B * NF * H * 4,
                 beta=dirs * B * T * H * 4, s_in=dirs * B * H * dv * dk * 4, s_out=dirs * B * H * dv * dk * 4,
                 out=B * T * H * dv * 4, gate=B * T * H * dv * es, nw=dv * 4, ws=1 << 30)
    addr, p = {}, BASE
    for k_, n in sizes.items():
        addr[k_] = p
        p += (n + 255) // 256 * 256 + 256
    return addr


def _call(prob, a, direction=gdn.GDN_DIR_FORWARD, **over):
    a = dict(a, **over)
    return gdn.gdn_vda_forward(prob, a["q"], a["k"], a["v"], a["la"], a["beta"], a["s_in"], a["s_out"], a["out"],
                               direction)


def _valid(direction=gdn.GDN_DIR_FORWARD, **kw):
    a = _bufs(dirs=2 if direction == gdn.GDN_DIR_BIDIRECTIONAL else 1)
    p = _prob(**kw)
    p.workspace = a["ws"]
    p.workspace_bytes = 1 << 30
    return p, a


def test_struct_layout_matches_c(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "gdn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(gdn_vda_problem_t),
         offsetof(gdn_vda_problem_t, frame), offsetof(gdn_vda_problem_t, dtype), offsetof(gdn_vda_problem_t, options),
         offsetof(gdn_vda_problem_t, readout_lag), offsetof(gdn_vda_problem_t, norm_eps),
         offsetof(gdn_vda_problem_t, gate), offsetof(gdn_vda_problem_t, norm_weight),
         offsetof(gdn_vda_problem_t, workspace), offsetof(gdn_vda_problem_t, workspace_bytes),
         offsetof(gdn_vda_problem_t, stream), offsetof(gdn_vda_problem_t, timing_events));
  printf("%d\\n", (int)GDN_VDA_OPT_ADDITIVE);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", f"-I{os.path.join(ROOT, 'include')}", str(prog), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)], text=True).split()]
    P = gdn.gdn_vda_problem_t
    assert got[:-1] == [ctypes_size(P), P.frame.offset, P.dtype.offset, P.options.offset, P.readout_lag.offset,
                        P.norm_eps.offset, P.gate.offset, P.norm_weight.offset, P.workspace.offset,
                        P.workspace_bytes.offset, P.stream.offset, P.timing_events.offset]
    assert got[-1] == gdn.GDN_VDA_OPT_ADDITIVE


def ctypes_size(P):
    import ctypes
    return ctypes.sizeof(P)


def test_workspace_bytes():
    one = gdn.gdn_vda_workspace_bytes(_prob(), gdn.GDN_DIR_FORWARD)
    two = gdn.gdn_vda_workspace_bytes(_prob(), gdn.GDN_DIR_BIDIRECTIONAL)
    # three fp32 matrices per frame, head and direction: 3 frames x 2 heads x 3 x 128 x 128 x 4 B
    assert one == 3 * 2 * 3 * 128 * 128 * 4
    assert two == 2 * one
    assert gdn.gdn_vda_workspace_bytes(_prob(T=301), gdn.GDN_DIR_FORWARD) > one  # a fourth, partial frame
    assert gdn.gdn_vda_workspace_bytes(_prob(T=0), gdn.GDN_DIR_FORWARD) == 0


@pytest.mark.parametrize("kw", [dict(dk=96), dict(dv=32), dict(frame=0), dict(dtype=7), dict(B=0), dict(T=-1),
                                dict(T=1 << 20, H=8)])
def test_workspace_bytes_rejects(kw):
    assert gdn.gdn_vda_workspace_bytes(_prob(**kw), gdn.GDN_DIR_FORWARD) == 0


def test_argument_checks():
    p, a = _valid()
    assert _call(p, a, direction=5) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert gdn.lib().gdn_vda_forward(None, a["q"], a["k"], a["v"], a["la"], a["beta"], None, None, a["out"], 0) \
        == gdn.GDN_ERR_INVALID_ARGUMENT
    for f in ("q", "k", "v", "la", "beta", "out"):
        assert _call(p, a, **{f: None}) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call(p, a, q=a["q"] + 8) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call(p, a, out=a["q"]) == gdn.GDN_ERR_INVALID_ARGUMENT  # out over an input
    p.workspace_bytes = 1024
    assert _call(p, a) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    p, a = _valid()
    p.options = 2
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p, a = _valid(dk=96)
    assert _call(p, a) == gdn.GDN_ERR_UNSUPPORTED


def test_option_and_epilogue_checks():
    p, a = _valid()
    p.readout_lag = -1
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p, a = _valid()
    p.gate = a["gate"]  # no norm weights
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.norm_weight = a["nw"]
    for eps in (-1e-6, float("nan"), float("inf")):
        p.norm_eps = eps
        assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.norm_eps = 1e-6
    p.gate = a["gate"] + 8  # misaligned
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.gate = a["gate"]
    assert _call(p, a, out=a["gate"]) == gdn.GDN_ERR_INVALID_ARGUMENT  # out over the gate
    assert _call(p, a, s_out=a["nw"]) == gdn.GDN_ERR_INVALID_ARGUMENT  # state_out over the weights


def test_valid_options_reach_the_launch():
    # every option combination passes validation (no GPU here: the launch reports the failure)
    for opts in (0, gdn.GDN_VDA_OPT_ADDITIVE):
        for lag in (0, 1, 1000):
            for epi in (False, True):
                p, a = _valid()
                p.options, p.readout_lag = opts, lag
                if epi:
                    p.gate, p.norm_weight, p.norm_eps = a["gate"], a["nw"], 1e-6
                assert _call(p, a) == gdn.GDN_ERR_HIP


def test_empty_sequence_without_state_output_is_a_no_op():
    p, a = _valid(T=0)
    assert _call(p, a, s_out=None) == gdn.GDN_OK


def test_valid_call_without_gpu_reports_launch_failure():
    p, a = _valid()
    assert _call(p, a) == gdn.GDN_ERR_HIP
