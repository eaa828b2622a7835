"""sa_compress_static, the entry point that allocates nothing: its workspace
is the library's static device array.  Called through the C ABI (ctypes)
with caller-allocated inputs and outputs, and compared with sa_compress on
the same inputs, bit for bit (the same kernels on the same workspace layout),
and with the fp64 oracle at the bf16 bar; two calls in a row, the second on
a smaller problem, so the second call runs on the array the first one left.
Sizes beyond the array are refused on the host."""
import ctypes

import numpy as np
import pytest

from oracle import sketch_batch
from synth import make_inputs
from tests.gpu_util import TOL, rel_errors, upload

pytestmark = pytest.mark.gpu


def _static_call(inp, dev, S, m, err):
    import torch

    from prototype_attention_compression_amd import _lib
    pb = _lib.problem(inp.R, inp.N, inp.d, inp.k, _lib.SA_BF16)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return _lib.raw_compress_static(pb, p(dev["H"]) if inp.N > 0 else None, p(dev["offsets"]), p(dev["mask"]),
                                    p(dev["Wk"]), p(dev["Wv"]), p(dev["P"]), p(S), p(m), p(err), stream)


def test_static_entry_matches_sa_compress_twice():
    import torch

    import prototype_attention_compression_amd as sa
    cases = [make_inputs([3000, 0, 17, 2500, 1], d=128, k=1024, seed=8100, mask_tail_frac=0.1, name="static_a"),
             make_inputs([700, 33], d=128, k=256, seed=8101, name="static_b")]
    for inp in cases:
        print(f"[case] static entry {inp.name} R={inp.R} N={inp.N} k={inp.k} d={inp.d}", flush=True)
        dev = upload(inp)
        S = torch.empty((inp.R, inp.k, inp.d), dtype=torch.float32, device="cuda")
        m = torch.empty((inp.R, inp.k), dtype=torch.float32, device="cuda")
        err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        assert _static_call(inp, dev, S, m, err) == sa.SA_OK
        torch.cuda.synchronize()
        S0, m0 = sa.compress(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], mask=dev["mask"],
                             return_mass=True)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(S, S0) and torch.equal(m, m0)
        Sref, mref = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask)
        mx, mean = rel_errors(S.cpu().numpy(), Sref)
        print(f"   S max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert mx <= TOL["bf16"][0] and mean <= TOL["bf16"][1]


def test_static_entry_errors():
    import torch

    import prototype_attention_compression_amd as sa
    from prototype_attention_compression_amd import _lib
    # beyond the static array: refused before any launch
    need = sa.workspace_size(1, 300_000, 128, 1024)
    assert need > _lib.STATIC_SCRATCH_BYTES
    pb = _lib.problem(1, 300_000, 128, 1024, _lib.SA_BF16)
    fake = ctypes.c_void_p(1 << 20)
    assert _lib.raw_compress_static(pb, fake, fake, None, fake, fake, fake, fake, None, None, None) == \
        sa.SA_E_WORKSPACE
    # broken offsets: zero sketches and the flag in device_error
    inp = make_inputs([250, 0, 350], d=128, k=512, seed=8200)
    dev = upload(inp)
    dev["offsets"] = torch.tensor([0, 250, 200, 600], dtype=torch.int64, device="cuda")
    S = torch.full((inp.R, 512, 128), 7.0, dtype=torch.float32, device="cuda")
    err = torch.zeros((1,), dtype=torch.int32, device="cuda")
    assert _static_call(inp, dev, S, None, err) == sa.SA_OK
    torch.cuda.synchronize()
    assert int(err.item()) & sa.SA_DEVICE_ERR_OFFSETS
    assert not S.any()
