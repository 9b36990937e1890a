"""Helpers shared by the GPU tests: move generator output to the device, run
libgdn through its C ABI binding, and compare against the oracle."""
import numpy as np

import oracle
import synth

# Tolerances: max |gpu - oracle| <= TOL * RMS(oracle), per tensor, over every
# compared element.  bf16 inputs: 2e-2; fp32 inputs: 1e-4.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_torch(x, device="cuda"):
    import torch

    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def run_gpu(inputs, direction, chunk=0, dv_tile=0, state_in="use", want_state=True, serial=False, erase=True,
            exclusive="none"):
    import torch

    import gated_delta_rule_scan_amd as gdn

    d = {k: to_torch(v) for k, v in inputs.items()}
    s_in = d["state_in"] if state_in == "use" else state_in
    out, s_out = gdn.forward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s_in, direction, chunk=chunk,
                             dv_tile=dv_tile, want_state=want_state, serial=serial, erase=erase,
                             exclusive=exclusive)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if s_out is None else s_out.cpu().numpy())


def rel_err(got, ref):
    """max |got - ref| / RMS(ref) (RMS floored to avoid 0/0 on all-zero refs)."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if ref.size else 0.0
    return err / max(rms, 1e-30), err, rms


def check(got, ref, tol, what=""):
    r, err, rms = rel_err(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert r <= tol, f"{what}: max abs err {err:.3e} = {r:.3e} x RMS {rms:.3e} > {tol:.1e} x RMS"
    return r
