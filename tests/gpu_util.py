"""Helpers for the GPU tests: upload synthetic inputs, run libsa through the
binding, and the normwise error measures used as the parity bar."""
import numpy as np

import prototype_attention_compression_amd as sa

# parity bar: bf16 inputs max_rel <= 2e-2 and mean_rel <= 2e-3; fp32 <= 1e-4
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}


def upload(inp, device="cuda"):
    import torch
    if inp.dtype == "bf16":
        def t(bits):
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
        H, Wk, Wv, P = t(inp.H_bits), t(inp.Wk_bits), t(inp.Wv_bits), t(inp.P_bits)
    else:
        def t(x):
            return torch.from_numpy(np.ascontiguousarray(x)).to(device)
        H, Wk, Wv, P = t(inp.H), t(inp.Wk), t(inp.Wv), t(inp.P)
    off = torch.from_numpy(inp.offsets).to(device)
    mask = None if inp.mask is None else torch.from_numpy(inp.mask).to(device)
    return dict(H=H, offsets=off, Wk=Wk, Wv=Wv, P=P, mask=mask)


def run(dev_inputs, return_mass=True, **kw):
    import torch
    S, m = sa.compress(dev_inputs["H"], dev_inputs["offsets"], dev_inputs["Wk"], dev_inputs["Wv"],
                       dev_inputs["P"], mask=dev_inputs["mask"], return_mass=True, **kw)
    torch.cuda.synchronize()
    return S, m


def rel_errors(S, ref):
    S = np.asarray(S, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(S - ref)
    denom_max = np.abs(ref).max()
    denom_sum = np.abs(ref).sum()
    if denom_max == 0:
        return float(diff.max()), float(diff.sum())
    return float(diff.max() / denom_max), float(diff.sum() / denom_sum)
