"""Seeded random sweep of problem shapes: GPU against the fp64 oracles.

Each case draws, from its own seed, a user count, ragged lengths (some users
empty, some a single token, some straddling tile and stage boundaries), k
(a multiple of 64 up to 2048), d (64 or 128), the input dtype and a tail
mask, and compares every user's sketch and mass with the oracle at the same
bar as the fixed parity tests (bf16: max_rel <= 2e-2, mean_rel <= 2e-3; fp32:
1e-4).  The backward cases compare all four gradients.  Sizes stay where the
oracle finishes each case in about a second."""
import numpy as np
import pytest

from oracle import sketch_batch, sketch_batch_grad
from synth import make_inputs, make_sketch_grad
from tests.gpu_util import TOL, rel_errors, run, upload

pytestmark = pytest.mark.gpu

K_CHOICES = [64, 128, 192, 256, 320, 512, 768, 1024, 2048]


def _draw(seed: int, bf16_only: bool = False):
    rng = np.random.default_rng(90000 + seed)
    R = int(rng.integers(1, 24))
    kinds = rng.integers(0, 5, size=R)
    lens = np.where(kinds == 0, 0,
                    np.where(kinds == 1, 1,
                             np.where(kinds == 2, rng.integers(2, 200, size=R), rng.integers(200, 6000, size=R))))
    if lens.sum() == 0:
        lens[0] = 257
    k = int(rng.choice(K_CHOICES))
    d = int(rng.choice([64, 128]))
    dtype = "bf16" if bf16_only or rng.random() < 0.8 else "f32"
    mask = float(rng.choice([0.0, 0.0, 0.15]))
    return [int(x) for x in lens], k, d, dtype, mask


@pytest.mark.parametrize("seed", range(16))
def test_forward_sweep(seed):
    lens, k, d, dtype, mask = _draw(seed)
    inp = make_inputs(lens, d=d, k=k, seed=91000 + seed, dtype=dtype, mask_tail_frac=mask, name=f"sweep{seed}")
    print(f"[case] sweep {seed}: R={inp.R} N={inp.N} k={k} d={d} dtype={dtype} mask={mask}", flush=True)
    S, m = run(upload(inp))
    S = S.cpu().numpy()
    m = m.cpu().numpy()
    Sref, mref = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask)
    tmax, tmean = TOL[dtype]
    mx, mean = rel_errors(S, Sref)
    mmx, mmean = rel_errors(m, mref)
    print(f"   S max_rel={mx:.3e} mean_rel={mean:.3e}  mass max_rel={mmx:.3e} mean_rel={mmean:.3e}", flush=True)
    assert np.isfinite(S).all() and np.isfinite(m).all()
    assert mx <= tmax and mean <= tmean, (mx, mean)
    assert mmx <= tmax and mmean <= tmean, (mmx, mmean)
    for u in range(inp.R):   # a user with no kept token gets exact zeros
        sl = inp.user_slice(u)
        n_kept = int(inp.lengths[u]) if inp.mask is None else int(inp.mask[sl].sum())
        if n_kept == 0:
            assert not S[u].any() and not m[u].any()


@pytest.mark.parametrize("seed", range(6))
def test_backward_sweep(seed):
    import torch

    import prototype_attention_compression_amd as sa
    lens, k, d, _, mask = _draw(100 + seed, bf16_only=True)
    inp = make_inputs(lens, d=d, k=k, seed=92000 + seed, mask_tail_frac=mask, name=f"bsweep{seed}")
    dS = make_sketch_grad(inp.R, k, d, seed=93000 + seed)
    print(f"[case] backward sweep {seed}: R={inp.R} N={inp.N} k={k} d={d} mask={mask}", flush=True)
    dev = upload(inp)
    out = sa.compress_backward(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"],
                               torch.from_numpy(dS).to("cuda"), mask=dev["mask"])
    torch.cuda.synchronize()
    dH, dP, dWk, dWv = [t.cpu().numpy() for t in out]
    ref = sketch_batch_grad(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, dS, mask=inp.mask)
    tmax, tmean = TOL["bf16"]
    for name, got, want in zip(("dH", "dP", "dWk", "dWv"), (dH, dP, dWk, dWv), ref):
        mx, mean = rel_errors(got, want)
        print(f"   {name} max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert np.isfinite(got).all()
        assert mx <= tmax and mean <= tmean, (name, mx, mean)
