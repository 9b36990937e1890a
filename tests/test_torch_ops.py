"""The torch.library custom ops (torch.ops.gdn.forward, torch.ops.gdn.vda_forward):
on the CPU, their fake implementations give the output shapes and an FX trace
with fake CUDA tensors keeps each call as one node; on the GPU, a
torch.compile'd function (fullgraph, no graph break) equals the eager calls."""
import pytest


def _fake_inputs(direction="bi", frame=None):
    import torch

    dirs = 2 if direction == "bi" else 1
    q = torch.empty((2, 300, 3, 64), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((2, 300, 3, 128), dtype=torch.bfloat16, device="cuda")
    nla = 300 if frame is None else -(-300 // frame)
    la = torch.empty((dirs, 2, nla, 3), device="cuda")
    bt = torch.empty((dirs, 2, 300, 3), device="cuda")
    return q, v, la, bt


@pytest.mark.parametrize("direction", ["fwd", "rev", "bi"])
def test_fake_shapes_and_trace(direction):
    import torch
    from torch._subclasses.fake_tensor import FakeTensorMode
    from torch.fx.experimental.proxy_tensor import make_fx

    import gated_delta_rule_scan_amd as gdn

    gdn.register_torch_ops()
    dirs = 2 if direction == "bi" else 1
    with FakeTensorMode():
        q, v, la, bt = _fake_inputs(direction)
        o, s = torch.ops.gdn.forward(q, q, v, la, bt, None, direction, 0, 0, True)
        assert tuple(o.shape) == (2, 300, 3, 128) and o.dtype == torch.float32
        assert tuple(s.shape) == (dirs, 2, 3, 128, 64) and s.dtype == torch.float32
        q2, v2, la2, bt2 = _fake_inputs(direction, frame=100)
        o, s = torch.ops.gdn.vda_forward(q2, q2, v2, la2, bt2, None, direction, 100, "additive", 1, None, None, 1e-6)
        assert tuple(o.shape) == (2, 300, 3, 128) and tuple(s.shape) == (dirs, 2, 3, 128, 64)

        def fn(q, v, la, bt):
            o, s = torch.ops.gdn.forward(q, q, v, la, bt, None, direction, 0, 0, True)
            return o * 2.0, s

        g = make_fx(fn, tracing_mode="fake")(q, v, la, bt)
    calls = [n for n in g.graph.nodes if n.op == "call_function" and "gdn" in str(n.target)]
    assert len(calls) == 1


@pytest.mark.gpu
def test_compiled_calls_equal_eager():
    import torch

    import gated_delta_rule_scan_amd as gdn
    import synth
    from gdn_testutil import to_torch

    gdn.register_torch_ops()
    w = synth.Workload("ops", 1, 2, 500, 128, 128, "bf16", "bi", 3.0, 0.02, 41)
    x = {k: to_torch(v) for k, v in synth.generate(w).items()}
    wf = synth.Workload("ops vda", 1, 2, 500, 128, 128, "bf16", "bi", -3.0, 0.05, 42)
    xf = {k: to_torch(v) for k, v in synth.generate_frames(wf, 100).items()}
    e = synth.generate_epilogue(wf)
    z, nw = to_torch(e["gate"]), to_torch(e["norm_weight"])

    def fn(x, xf, z, nw):
        o, s = torch.ops.gdn.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi", 0, 0, True)
        of, sf = torch.ops.gdn.vda_forward(xf["q"], xf["k"], xf["v"], xf["log_alpha"], xf["beta"], xf["state_in"], "bi",
                                           100, "inverse", 2, z, nw, 1e-6)
        return o + 1.0, s, of, sf

    compiled = torch.compile(fn, backend="aot_eager", fullgraph=True)
    got = compiled(x, xf, z, nw)
    o, s = gdn.forward(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], x["state_in"], "bi")
    of, sf = gdn.vda_forward(xf["q"], xf["k"], xf["v"], xf["log_alpha"], xf["beta"], xf["state_in"], "bi", 100, lag=2,
                             gate=z, norm_weight=nw, norm_eps=1e-6)
    torch.cuda.synchronize()
    for a, b in zip(got, (o + 1.0, s, of, sf)):
        assert torch.equal(a, b)
