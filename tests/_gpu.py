"""Helpers shared by the GPU tests: move a synthetic layer to the device, run
the HIP library through its C ABI, and compare with the oracle."""
import math

import numpy as np
import torch

import weight_only_bit_moe_amd as M

#: Elementwise bound for the layer output: |gpu - oracle| <= REL * rms(oracle) + ABS,
#: with rms over every output element compared.
REL, ABS = 2e-2, 1e-3


def device():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_device(L, dev):
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(
        x=torch.from_numpy(L.x.view(np.int16)).to(dev).view(torch.bfloat16),
        topk_ids=t(L.topk_ids, np.int32),
        topk_w=t(L.topk_w, np.float32),
        w13=torch.from_numpy(L.w13.view(np.int32)).to(dev),
        s13=torch.from_numpy(L.s13).to(dev),
        w2=torch.from_numpy(L.w2.view(np.int32)).to(dev),
        s2=torch.from_numpy(L.s2).to(dev),
    )


def run_layer(L, dev, d=None, out=None, workspace=None):
    sp = L.spec
    d = d or to_device(L, dev)
    clamp = None if math.isinf(sp.clamp) else sp.clamp
    y = M.forward(d["x"], d["topk_ids"], d["topk_w"], d["w13"], d["s13"], d["w2"], d["s2"],
                  bits=(sp.bits13, sp.bits2), group=(sp.group13, sp.group2), alpha=sp.alpha,
                  beta=sp.beta, clamp=clamp, out=out, workspace=workspace)
    torch.cuda.synchronize(dev)
    return y


def to_f64(y):
    return y.float().cpu().numpy().astype(np.float64)


def parity_ratio(got, ref):
    """max |got - ref| / (REL * rms(ref) + ABS) over all compared elements."""
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    tol = REL * rms + ABS
    return float(np.max(np.abs(got - ref))) / tol if ref.size else 0.0


def assert_parity(got, ref, what=""):
    r = parity_ratio(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert r <= 1.0, f"{what}: max error is {r:.3f}x the tolerance"
    return r
