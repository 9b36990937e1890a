"""The libgdn C ABI on the host (no kernel runs here): exported symbols match
include/gdn.h, the ctypes mirror of gdn_problem_t matches the C layout, and
every argument check returns its status before anything is enqueued.

A fully valid call on a machine without a GPU reaches the kernel launch and
must report GDN_ERR_HIP (the launch-failure path)."""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_scan_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_exported_entry_points():
    assert _declared_functions() == sorted(gdn.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = gdn.lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.check_output(["nm", "-D", "--defined-only", gdn.LIB_PATH], text=True)
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(_declared_functions()) <= exported


def test_problem_struct_layout_matches_c(tmp_path):
    prog = tmp_path / "layout.c"
    prog.write_text("""
#include <stdio.h>
#include <stddef.h>
#include "gdn.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %d %d %d %d %d\\n", sizeof(gdn_problem_t),
         offsetof(gdn_problem_t, dtype),
         offsetof(gdn_problem_t, chunk), offsetof(gdn_problem_t, dv_tile), offsetof(gdn_problem_t, options),
         offsetof(gdn_problem_t, workspace),
         offsetof(gdn_problem_t, workspace_bytes), offsetof(gdn_problem_t, stream),
         offsetof(gdn_problem_t, timing_events), offsetof(gdn_problem_t, gate), offsetof(gdn_problem_t, norm_weight),
         offsetof(gdn_problem_t, norm_eps), (int)GDN_OPT_SERIAL, (int)GDN_OPT_NO_ERASE,
         (int)GDN_OPT_EXCLUSIVE_FORWARD, (int)GDN_OPT_EXCLUSIVE_REVERSE, (int)GDN_OPT_TEST_NO_PREPARATION);
  return 0;
}
""")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", f"-I{os.path.join(ROOT, 'include')}", str(prog), "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)], text=True).split()]
    P = gdn.gdn_problem_t
    want = [ctypes.sizeof(P), P.dtype.offset, P.chunk.offset, P.dv_tile.offset, P.options.offset, P.workspace.offset,
            P.workspace_bytes.offset, P.stream.offset, P.timing_events.offset, P.gate.offset, P.norm_weight.offset,
            P.norm_eps.offset, gdn.GDN_OPT_SERIAL, gdn.GDN_OPT_NO_ERASE,
            gdn.GDN_OPT_EXCLUSIVE_FORWARD, gdn.GDN_OPT_EXCLUSIVE_REVERSE, gdn.GDN_OPT_TEST_NO_PREPARATION]
    assert got == want


def test_version_and_status_strings():
    assert "gfx950" in gdn.gdn_version()
    assert gdn.gdn_status_string(gdn.GDN_OK) == "ok"
    for st in range(1, 5):
        assert gdn.gdn_status_string(st) not in ("ok", "unknown status")
    assert gdn.gdn_status_string(99) == "unknown status"


def _prob(B=1, T=300, H=2, dk=128, dv=128, dtype=gdn.GDN_DTYPE_BF16, chunk=0, dv_tile=0, ws=0, wsb=0):
    return gdn.make_problem(B, T, H, dk, dv, dtype, chunk, dv_tile, ws, wsb)


def test_workspace_bytes():
    for d in ("fwd", "rev", "bi"):
        assert gdn.workspace_bytes(1, 300, 2, 128, 128, "bf16", d) > 0
    n1 = gdn.workspace_bytes(1, 300, 2, 128, 128, "bf16", "fwd")
    n2 = gdn.workspace_bytes(1, 300, 2, 128, 128, "bf16", "bi")
    assert n2 > n1
    assert gdn.workspace_bytes(1, 300, 2, 64, 64, "f32", "fwd") > gdn.workspace_bytes(1, 300, 2, 64, 64, "bf16", "fwd")
    # chunk count rounds up: one token more than a chunk multiple needs one chunk more
    assert gdn.workspace_bytes(1, 129, 1, 64, 64, "bf16", "fwd") > gdn.workspace_bytes(1, 128, 1, 64, 64, "bf16", "fwd")
    assert gdn.workspace_bytes(1, 0, 1, 64, 64, "bf16", "fwd") == 0  # an empty sequence needs none


def test_workspace_bytes_of_exclusive_readouts():
    """bf16 exclusive readouts also keep the low parts of the decayed q.k
    tile: C x C bf16 per chunk and head (C = 64 here, 5 chunks, 2 heads);
    fp32 operands need nothing more."""
    for ex in ("fwd", "rev", "both"):
        extra = (gdn.workspace_bytes(1, 300, 2, 128, 128, "bf16", "bi", exclusive=ex)
                 - gdn.workspace_bytes(1, 300, 2, 128, 128, "bf16", "bi"))
        assert 5 * 2 * 64 * 64 * 2 <= extra < 5 * 2 * 64 * 64 * 2 + 256
        assert (gdn.workspace_bytes(1, 300, 2, 64, 64, "f32", "bi", exclusive=ex)
                == gdn.workspace_bytes(1, 300, 2, 64, 64, "f32", "bi"))


@pytest.mark.parametrize("kw", [dict(dk=96), dict(dv=80), dict(chunk=48), dict(chunk=8), dict(chunk=256), dict(dv_tile=64),
                                dict(dtype=7), dict(B=0), dict(H=0), dict(T=-1), dict(B=300, H=300),
                                dict(dv_tile=48), dict(T=1 << 20, H=8, dk=128, dv=128)])
def test_workspace_bytes_rejects(kw):
    assert gdn.gdn_workspace_bytes(_prob(**kw), gdn.GDN_DIR_FORWARD) == 0


def test_workspace_bytes_rejects_bad_direction():
    assert gdn.gdn_workspace_bytes(_prob(), 3) == 0
    assert gdn.gdn_workspace_bytes(_prob(), -1) == 0


# Fake, well-aligned device addresses: validation never dereferences them.
BASE = 1 << 40


def _bufs(B=1, T=300, H=2, dk=128, dv=128, es=2, dirs=1):
    """Disjoint fake buffers laid out one after another (256-byte aligned)."""
    sizes = dict(q=B * T * H * dk * es, k=B * T * H * dk * es, v=B * T * H * dv * es, la=dirs * B * T * H * 4,
                 beta=dirs * B * T * H * 4, s_in=dirs * B * H * dv * dk * 4, s_out=dirs * B * H * dv * dk * 4,
                 out=B * T * H * dv * 4, ws=1 << 30)
    addr, p = {}, BASE
    for k_, n in sizes.items():
        addr[k_] = p
        p += (n + 255) // 256 * 256 + 256
    return addr


def _call(prob, a, direction=gdn.GDN_DIR_FORWARD, **over):
    a = dict(a, **over)
    return gdn.gdn_forward(prob, a["q"], a["k"], a["v"], a["la"], a["beta"], a["s_in"], a["s_out"], a["out"],
                           direction)


def _valid(direction=gdn.GDN_DIR_FORWARD, **kw):
    a = _bufs(dirs=2 if direction == gdn.GDN_DIR_BIDIRECTIONAL else 1)
    p = _prob(**kw)
    p.workspace = a["ws"]
    p.workspace_bytes = 1 << 30
    return p, a


def test_null_problem_is_invalid():
    a = _bufs()
    st = gdn.lib().gdn_forward(None, a["q"], a["k"], a["v"], a["la"], a["beta"], None, None, a["out"], 0)
    assert st == gdn.GDN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field", ["q", "k", "v", "la", "beta", "out"])
def test_null_required_pointer_is_invalid(field):
    p, a = _valid()
    assert _call(p, a, **{field: None}) == gdn.GDN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("field,offset", [("q", 8), ("k", 2), ("v", 4), ("out", 8), ("la", 2), ("s_in", 4),
                                          ("s_out", 8)])
def test_misaligned_pointer_is_invalid(field, offset):
    p, a = _valid()
    assert _call(p, a, **{field: a[field] + offset}) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_workspace_checks():
    p, a = _valid()
    need = gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_FORWARD)
    p.workspace_bytes = need - 1
    assert _call(p, a) == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    p.workspace_bytes = need
    p.workspace = a["ws"] + 128
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.workspace = None
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_overlaps_are_invalid():
    p, a = _valid()
    assert _call(p, a, out=a["q"]) == gdn.GDN_ERR_INVALID_ARGUMENT           # out aliases an input
    assert _call(p, a, out=a["v"] + 256) == gdn.GDN_ERR_INVALID_ARGUMENT     # partial overlap
    assert _call(p, a, s_out=a["k"]) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call(p, a, s_out=a["s_in"] + 256) == gdn.GDN_ERR_INVALID_ARGUMENT  # partial state overlap
    p.workspace = a["out"]
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT                       # workspace over out


def test_bad_problem_fields():
    p, a = _valid()
    assert _call(p, a, direction=5) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.options = 16  # undefined option bit
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.options = -1
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p.options = 1 << 17
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    # the test option needs the ready-flag path, which the serial order does not take
    p.options = gdn.GDN_OPT_TEST_NO_PREPARATION | gdn.GDN_OPT_SERIAL
    assert _call(p, a) == gdn.GDN_ERR_INVALID_ARGUMENT
    p, a = _valid(dk=96)
    assert _call(p, a) == gdn.GDN_ERR_UNSUPPORTED
    p, a = _valid(chunk=48)
    assert _call(p, a) == gdn.GDN_ERR_UNSUPPORTED


def test_empty_sequence_without_state_output_is_a_no_op():
    p, a = _valid(T=0)
    assert _call(p, a, q=None, k=None, v=None, la=None, beta=None, out=None, s_out=None) == gdn.GDN_OK


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU is present: the launch would succeed")
@pytest.mark.parametrize("direction", [gdn.GDN_DIR_FORWARD, gdn.GDN_DIR_REVERSE, gdn.GDN_DIR_BIDIRECTIONAL])
def test_valid_call_without_gpu_reports_launch_failure(direction):
    p, a = _valid(direction)
    assert _call(p, a, direction) == gdn.GDN_ERR_HIP
    # state_in == state_out (in-place carry) passes validation too
    assert _call(p, a, direction, s_out=a["s_in"]) == gdn.GDN_ERR_HIP
    # so does every combination of defined option bits
    for opts in range(16):
        p.options = opts
        assert _call(p, a, direction) == gdn.GDN_ERR_HIP
    p.options = gdn.GDN_OPT_TEST_NO_PREPARATION
    assert _call(p, a, direction) == gdn.GDN_ERR_HIP


def test_binding_raises_on_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        gdn.lib()


def test_size_limits_are_exact():
    """The documented limits, checked on both sides: B*H <= 65535, and one
    batch element's rows, (T + 64) * H * max(dk, dv) * 4 bytes, below 2^32."""
    ws = lambda B, T, H, d=128, direction="bi": gdn.workspace_bytes(B, T, H, d, d, "bf16", direction)
    assert ws(3, 5, 21845) > 0            # B*H = 65535
    assert ws(1, 5, 65536) == 0
    assert ws(65535, 5, 1) > 0
    assert ws(2, 5, 32768) == 0
    t_max = (1 << 32) // (128 * 4) - 64 - 1  # 8,388,543 tokens at H = 1, d = 128
    assert ws(1, t_max, 1) > 0
    assert ws(1, t_max + 1, 1) == 0
    t_max64 = (1 << 32) // (64 * 4) - 64 - 1
    assert gdn.workspace_bytes(1, t_max64, 1, 64, 64, "f32", "fwd") > 0
    assert gdn.workspace_bytes(1, t_max64 + 1, 1, 64, 64, "f32", "fwd") == 0
    # the same limits through gdn_forward (no GPU needed: rejected before any launch)
    p, a = _valid(T=t_max + 1, H=1, dk=128, dv=128)
    assert _call(p, a) == gdn.GDN_ERR_UNSUPPORTED
    p, a = _valid(B=1, H=65536)
    assert _call(p, a) == gdn.GDN_ERR_UNSUPPORTED


def test_noalloc_limit_in_header_matches_binding():
    src = open(HEADER).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_problems_beyond_its_scratch_before_any_launch():
    """A problem whose workspace exceeds the fixed scratch is refused with
    GDN_ERR_WORKSPACE_TOO_SMALL before anything touches a device (this host
    has none); one that fits passes that check."""
    big = gdn.make_problem(2, 32760, 16, 128, 128, gdn.GDN_DTYPE_BF16)
    assert gdn.gdn_workspace_bytes(big, gdn.GDN_DIR_BIDIRECTIONAL) > gdn.NOALLOC_SCRATCH_BYTES
    fake = 1 << 40  # never dereferenced: the call returns before any launch
    st = gdn.gdn_forward_noalloc(big, fake, fake + (1 << 32), fake + (2 << 32), fake + (3 << 32), fake + (4 << 32),
                                 None, None, fake + (5 << 32), gdn.GDN_DIR_BIDIRECTIONAL)
    assert st == gdn.GDN_ERR_WORKSPACE_TOO_SMALL
    small = gdn.make_problem(1, 1560, 12, 128, 128, gdn.GDN_DTYPE_BF16)
    assert 0 < gdn.gdn_workspace_bytes(small, gdn.GDN_DIR_FORWARD) <= gdn.NOALLOC_SCRATCH_BYTES
    # invalid arguments are still reported first
    assert gdn.gdn_forward_noalloc(small, None, None, None, None, None, None, None, None,
                                   gdn.GDN_DIR_FORWARD) == gdn.GDN_ERR_INVALID_ARGUMENT


def test_exclusive_bf16_rejects_32_wide_tiles():
    """bf16 exclusive readouts run 16-column tiles only (the state's and the
    q.k tile's low parts fit that staging): an explicit 32 is unsupported,
    before anything is enqueued; fp32 and inclusive bf16 accept it."""
    p = _prob(dv_tile=32)
    p.options = gdn.GDN_OPT_EXCLUSIVE_FORWARD
    assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_FORWARD) == 0
    p.options = 0
    assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_FORWARD) > 0
    p = _prob(dv_tile=32, dtype=gdn.GDN_DTYPE_F32)
    p.options = gdn.GDN_OPT_EXCLUSIVE_FORWARD
    assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_FORWARD) > 0


def test_epilogue_arguments_are_validated_before_launch():
    """The readout epilogue's arguments: a gate needs a norm weight, both
    16-byte aligned, a finite non-negative eps, and `out` may not overlap
    either; all rejected before anything is enqueued.  Valid ones reach the
    launch (which fails here, with no GPU)."""
    p, a = _valid()
    end = max(a.values()) + (1 << 30) + 4096  # past the fake workspace
    gate, nw = end, end + 300 * 2 * 128 * 2 + 256

    def with_epi(g=gate, w=nw, eps=1e-6):
        q, _ = _valid()
        q.gate, q.norm_weight, q.norm_eps = g, w, eps
        return q

    assert _call(with_epi(w=None), a) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call(with_epi(g=gate + 8), a) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call(with_epi(w=nw + 4), a) == gdn.GDN_ERR_INVALID_ARGUMENT
    for eps in (-1e-6, float("nan"), float("inf")):
        assert _call(with_epi(eps=eps), a) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call(with_epi(g=a["out"]), a) == gdn.GDN_ERR_INVALID_ARGUMENT  # gate overlaps out
    assert _call(with_epi(w=a["out"] + 512), a) == gdn.GDN_ERR_INVALID_ARGUMENT  # weights inside out
    assert _call(with_epi(), a) == gdn.GDN_ERR_HIP
    assert _call(with_epi(eps=0.0), a) == gdn.GDN_ERR_HIP
    # an invalid epilogue also makes the workspace query fail
    assert gdn.gdn_workspace_bytes(with_epi(w=None), gdn.GDN_DIR_FORWARD) == 0


def test_chunk128_is_accepted_with_its_limits():
    """128-token chunks: accepted for both operand types in every direction;
    the workspace holds C x C triangles per chunk (3 chunks of 300 tokens);
    bf16 exclusive readouts and the bf16 epilogue (whose low parts only the
    32/64-token chain carries) and 32-wide fp32 tiles at d = 128 (their
    staging exceeds the compute unit's LDS) are unsupported, rejected before
    anything is enqueued."""
    for dtype in (gdn.GDN_DTYPE_BF16, gdn.GDN_DTYPE_F32):
        for d in (gdn.GDN_DIR_FORWARD, gdn.GDN_DIR_REVERSE, gdn.GDN_DIR_BIDIRECTIONAL):
            assert gdn.gdn_workspace_bytes(_prob(chunk=128, dtype=dtype), d) > 0
    es = 2
    assert gdn.gdn_workspace_bytes(_prob(chunk=128), gdn.GDN_DIR_FORWARD) >= 2 * 3 * 2 * 128 * 128 * es
    for opt in (gdn.GDN_OPT_EXCLUSIVE_FORWARD, gdn.GDN_OPT_EXCLUSIVE_REVERSE):
        p = _prob(chunk=128)
        p.options = opt
        assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_BIDIRECTIONAL) == 0
        p = _prob(chunk=128, dtype=gdn.GDN_DTYPE_F32)
        p.options = opt
        assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_BIDIRECTIONAL) > 0
    for dtype, want in ((gdn.GDN_DTYPE_BF16, False), (gdn.GDN_DTYPE_F32, True)):
        p = _prob(chunk=128, dtype=dtype)
        p.gate, p.norm_weight, p.norm_eps = 1 << 40, 1 << 41, 1e-6  # host-side validation only
        assert (gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_FORWARD) > 0) == want
    assert gdn.gdn_workspace_bytes(_prob(chunk=128, dtype=gdn.GDN_DTYPE_F32, dv_tile=32), gdn.GDN_DIR_FORWARD) == 0
    assert gdn.gdn_workspace_bytes(_prob(chunk=128, dtype=gdn.GDN_DTYPE_F32, dk=64, dv=64, dv_tile=32),
                                   gdn.GDN_DIR_FORWARD) > 0
    assert gdn.gdn_workspace_bytes(_prob(chunk=128, dv_tile=32), gdn.GDN_DIR_FORWARD) > 0


def test_chunk16_is_accepted_with_its_limits():
    """16-token chunks: accepted for both operand types in every direction;
    bf16 exclusive readouts and the bf16 epilogue are unsupported there (as at
    128 tokens), fp32 takes every option."""
    for dtype in (gdn.GDN_DTYPE_BF16, gdn.GDN_DTYPE_F32):
        for d in (gdn.GDN_DIR_FORWARD, gdn.GDN_DIR_REVERSE, gdn.GDN_DIR_BIDIRECTIONAL):
            assert gdn.gdn_workspace_bytes(_prob(chunk=16, dtype=dtype), d) > 0
        for dv_tile in (16, 32):
            assert gdn.gdn_workspace_bytes(_prob(chunk=16, dtype=dtype, dv_tile=dv_tile), gdn.GDN_DIR_FORWARD) > 0
    # 19 chunks of 300 tokens, 2 heads: the triangles are 16 x 16 per chunk
    assert gdn.gdn_workspace_bytes(_prob(chunk=16), gdn.GDN_DIR_FORWARD) >= 2 * 19 * 2 * 16 * 16 * 2
    p = _prob(chunk=16)
    p.options = gdn.GDN_OPT_EXCLUSIVE_FORWARD
    assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_BIDIRECTIONAL) == 0
    p = _prob(chunk=16, dtype=gdn.GDN_DTYPE_F32)
    p.options = gdn.GDN_OPT_EXCLUSIVE_FORWARD
    assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_BIDIRECTIONAL) > 0
    p = _prob(chunk=16)
    p.gate, p.norm_weight, p.norm_eps = 1 << 40, 1 << 41, 1e-6  # host-side validation only
    assert gdn.gdn_workspace_bytes(p, gdn.GDN_DIR_FORWARD) == 0
