"""GPU parity of the backward pass (sa_compress_backward) against the fp64
gradient oracle on the same seeded inputs.

Bar: the four gradients (dH of the compared tokens, dP, dWk, dWv) each within
max_rel <= 2e-2 and mean_rel <= 2e-3 (normwise, as for the sketches): the
kernels use fp16 MFMA operands (queries rounded to fp16, allocations and
their gradients scaled into fp16 range) with fp32 sums.  Full-size
workloads use the linearity of the gradients in dS: dS is nonzero only for a
sample of users, so the oracle needs only those users, the parameter
gradients are exactly their sum, and every other user's dH must be exactly
zero."""
import numpy as np
import pytest

from oracle import normalised_rows_batch, sketch_batch, sketch_batch_grad
from synth import make_config, make_inputs, make_sketch_grad
from tests.gpu_util import TOL, rel_errors, upload

pytestmark = pytest.mark.gpu


def _run(dev, dS):
    import torch

    import prototype_attention_compression_amd as sa
    out = sa.compress_backward(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"],
                               torch.from_numpy(dS).to("cuda"), mask=dev["mask"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _check(inp, dS, users=None, tol=None):
    """Compare all four gradients; ``users``: dS is zero outside these."""
    print(f"[case] backward {inp.name} R={inp.R} N={inp.N} k={inp.k} d={inp.d} users={users} "
          f"|dS|max={np.abs(dS).max():.3g}", flush=True)
    dev = upload(inp)
    dH, dP, dWk, dWv = _run(dev, dS)
    if users is None:
        ref = sketch_batch_grad(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, dS, mask=inp.mask)
        rows = np.arange(inp.N)
    else:
        sel = sorted(users)
        lens = [int(inp.offsets[u + 1] - inp.offsets[u]) for u in sel]
        off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
        rows = np.concatenate([np.arange(inp.offsets[u], inp.offsets[u + 1]) for u in sel])
        mask = None if inp.mask is None else inp.mask[rows]
        ref = sketch_batch_grad(inp.H[rows], off, inp.Wk, inp.Wv, inp.P, dS[sel], mask=mask)
        other = np.ones(inp.N, dtype=bool)
        other[rows] = False
        assert not dH[other].any(), "dH of users with zero dS must be exactly zero"
    tmax, tmean = tol or TOL["bf16"]
    got = (dH[rows], dP, dWk, dWv)
    for name, g, r in zip(("dH", "dP", "dWk", "dWv"), got, ref):
        mx, mean = rel_errors(g, r)
        print(f"   {name}: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert np.isfinite(g).all(), name
        assert mx <= tmax and mean <= tmean, (name, mx, mean)
    if inp.mask is not None:
        assert not dH[inp.mask == 0].any(), "dropped tokens get zero rows"
    return dH, dP, dWk, dWv


@pytest.mark.parametrize("k", [64, 320, 1024, 2048])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_small_ragged(k, d):
    """Empty, one-token and tile-straddling users; several tiles per user,
    every prototype-block count from 1 (k = 64 at d = 64) up."""
    inp = make_inputs([0, 1, 31, 33, 700, 2049, 4], d=d, k=k, seed=4000 + k + d, name=f"bwd_k{k}_d{d}")
    _check(inp, make_sketch_grad(inp.R, k, d, seed=5000 + k + d))


def test_backward_one_token_users():
    """A user of one token has the sketch row h Wv for every prototype,
    whatever P and Wk, so it adds nothing to dP and dWk.  With many such users
    beside one long user those two gradients must equal what the long user
    gives alone, up to fp32 summation order (bar: mean_rel 1e-4, max_rel
    1e-3).  This holds only if each row's mean term c_j = Zs_j . Sbar_j is
    formed from the same fp16-rounded Z row as the per-token products
    Zs_j . h_t: with c from the unrounded row, every one-token user adds the
    fp16 rounding of Zs_j . h_t (about 5e-4 of it) where the exact value is 0."""
    import dataclasses
    lens = [1] * 24 + [1500] + [1] * 8
    inp = make_inputs(lens, d=128, k=256, seed=4700, name="bwd_one_token")
    dS = make_sketch_grad(inp.R, 256, 128, seed=5700)
    dH, dP, dWk, _ = _check(inp, dS)
    sl = inp.user_slice(24)
    alone = dataclasses.replace(inp, name="bwd_one_token_alone", lengths=np.array([1500], dtype=np.int64),
                                offsets=np.array([0, 1500], dtype=np.int64), H=inp.H[sl], H_bits=inp.H_bits[sl])
    dH1, dP1, dWk1, _ = _run(upload(alone), np.ascontiguousarray(dS[24:25]))
    for name, g, r in (("dP", dP, dP1), ("dWk", dWk, dWk1), ("dH", dH[sl], dH1)):
        mx, mean = rel_errors(g, r)
        print(f"   {name} batch vs alone: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert mx <= 1e-3 and mean <= 1e-4, (name, mx, mean)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_largest_k(d):
    """k = 4096, the largest built: 128 prototype blocks per token sweep,
    32 prototype-major workgroups per group."""
    inp = make_inputs([1500, 0, 33, 700], d=d, k=4096, seed=4900 + d, name=f"bwd_k4096_d{d}")
    _check(inp, make_sketch_grad(inp.R, 4096, d, seed=5900 + d))


@pytest.mark.parametrize("scale", [1e-7, 1e-2, 1e5])
def test_backward_dS_scale(scale):
    """The per-user and per-token power-of-two scales keep the fp16 operands
    in range whatever the size of dS."""
    inp = make_inputs([900, 0, 1500], d=128, k=512, seed=4100, name="bwd_scale")
    _check(inp, make_sketch_grad(inp.R, 512, 128, seed=5100, scale=scale))


def test_backward_masked_tokens():
    inp = make_inputs([1000, 1777, 64, 5], d=128, k=512, seed=4200, mask_tail_frac=0.3, name="bwd_mask")
    _check(inp, make_sketch_grad(inp.R, 512, 128, seed=5200))


@pytest.mark.parametrize("d,k", [(128, 1024), (64, 512)])
def test_backward_sharp_softmax(d, k):
    """Peaked softmax: P scaled by 4 sqrt(d), the forward's sharp config
    (logit std about 4), so the per-token power-of-two scales, the softmax
    Jacobian's centring and the fp16 scaling of dL work far from the uniform
    allocation of the Gaussian workloads."""
    from oracle import allocations, logits
    inp = make_inputs([3000, 1000], d=d, k=k, seed=4300 + d, p_scale=4.0 * np.sqrt(d), name=f"bwd_sharp_d{d}")
    A = allocations(logits(inp.H[:3000], inp.Wk, inp.P))
    top = float(A.max(axis=0).mean())
    print(f"   mean largest allocation per token {top:.3f} (uniform: {1.0 / k:.2e})", flush=True)
    assert top > 50.0 / k
    _check(inp, make_sketch_grad(inp.R, k, d, seed=5300 + d))


def test_backward_many_short_users():
    """Many users per group range in the prototype-major kernel (user
    boundaries inside a workgroup's range rescale E)."""
    rng = np.random.default_rng(4400)
    lens = rng.integers(0, 300, size=150)
    lens[::13] = 0
    inp = make_inputs(lens.tolist(), d=128, k=1024, seed=4401, name="bwd_many")
    # very different dS scales per user
    dS = make_sketch_grad(inp.R, 1024, 128, seed=5400)
    dS *= (10.0 ** rng.uniform(-3, 3, size=inp.R)).astype(np.float32)[:, None, None]
    _check(inp, dS)


def test_backward_deterministic():
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([3000, 17, 2500], d=128, k=1024, seed=4500)
    dev = upload(inp)
    dS = torch.from_numpy(make_sketch_grad(inp.R, 1024, 128, seed=5500)).to("cuda")
    a = sa.compress_backward(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], dS)
    b = sa.compress_backward(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], dS)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_empty_batches():
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([0, 0, 0], d=128, k=512, seed=4600)
    dev = upload(inp)
    dS = torch.ones((3, 512, 128), device="cuda")
    dH, dP, dWk, dWv = sa.compress_backward(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], dS)
    assert dH.shape == (0, 128)
    for t in (dP, dWk, dWv):
        assert not t.any()
    off0 = torch.zeros(1, dtype=torch.int64, device="cuda")
    dH, dP, dWk, dWv = sa.compress_backward(dev["H"], off0, dev["Wk"], dev["Wv"], dev["P"],
                                            torch.zeros((0, 512, 128), device="cuda"))
    for t in (dP, dWk, dWv):
        assert not t.any()


def test_backward_bad_offsets_zero_gradients():
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([250, 0, 350], d=128, k=512, seed=4700)
    dev = upload(inp)
    bad = torch.tensor([0, 250, 200, 600], dtype=torch.int64, device="cuda")
    dS = torch.from_numpy(make_sketch_grad(inp.R, 512, 128, seed=5700)).to("cuda")
    ws = torch.empty(sa.backward_workspace_size(inp.R, inp.N, 128, 512), dtype=torch.uint8, device="cuda")
    dH, dP, dWk, dWv = sa.compress_backward(dev["H"], bad, dev["Wk"], dev["Wv"], dev["P"], dS, workspace=ws)
    assert sa.read_device_error(ws) & sa.SA_DEVICE_ERR_OFFSETS
    for t in (dH, dP, dWk, dWv):
        assert not t.any()


def test_backward_bench_workload_sampled():
    """40 users x 100,000 tokens, k = 1024, d = 128 (the bench's workload and
    launch configuration), dS nonzero for users 0 and 23."""
    inp = make_config("c3lit_r40_n100k_d128_k1024")
    users = [0, 23]
    _check(inp, make_sketch_grad(inp.R, inp.k, inp.d, seed=5800, users=users), users=users)


def test_backward_ragged_training_batch_sampled():
    inp = make_config("c3_r40_ragged_d128_k1024")
    users = [int(np.argmin(inp.lengths)), int(np.argmax(inp.lengths))]
    _check(inp, make_sketch_grad(inp.R, inp.k, inp.d, seed=5900, users=users), users=users)


# ------------------------------------------------ the forward's state handed to the backward
@pytest.mark.parametrize("d,k", [(64, 320), (128, 1024)])
def test_forward_sbar_matches_oracle(d, k):
    """sa_compress_with_sbar: S and mass equal sa_compress's bit for bit, and
    Sbar matches the oracle's mass-normalised rows (same bar as S)."""
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([0, 1, 700, 2049, 33], d=d, k=k, seed=6000 + d, mask_tail_frac=0.1, name=f"sbar_d{d}")
    print(f"[case] forward with Sbar R={inp.R} N={inp.N} k={k} d={d}", flush=True)
    dev = upload(inp)
    args = (dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"])
    S0, m0 = sa.compress(*args, mask=dev["mask"], return_mass=True)
    S, m, Sbar = sa.compress(*args, mask=dev["mask"], return_sbar=True)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and torch.equal(m, m0)
    ref = normalised_rows_batch(inp.H, inp.offsets, inp.Wk, inp.P, mask=inp.mask)
    mx, mean = rel_errors(Sbar.cpu().numpy(), ref)
    print(f"   Sbar: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
    tmax, tmean = TOL["bf16"]
    assert mx <= tmax and mean <= tmean
    Sref, _ = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask)
    mx, mean = rel_errors(Sbar.cpu().numpy().astype(np.float64) @ inp.Wv, Sref)
    assert mx <= tmax and mean <= tmean
    assert not Sbar[0].any() and not m[0].any()    # the empty user


@pytest.mark.parametrize("d,k,lengths", [(64, 320, (3000, 0, 17, 2500, 1)), (128, 1024, (3000, 0, 17, 2500, 1)),
                                          (128, 1024, (60000, 5))])
def test_backward_with_sbar_equals_recompute(d, k, lengths):
    """sa_compress_backward_with_sbar on the forward's Sbar and masses gives
    the same gradients, bit for bit, as the backward that recomputes the
    per-user sums (the same fixed-order sums and divisions either way, also
    when a long user's slots are pre-summed), and they meet the gradient
    oracle's bar."""
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs(list(lengths), d=d, k=k, seed=6100 + d, mask_tail_frac=0.1, name=f"sbar_bwd_d{d}")
    print(f"[case] backward with Sbar R={inp.R} N={inp.N} k={k} d={d}", flush=True)
    dev = upload(inp)
    args = (dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"])
    dS_np = make_sketch_grad(inp.R, k, d, seed=6200 + d)
    dS = torch.from_numpy(dS_np).to("cuda")
    ref = sa.compress_backward(*args, dS, mask=dev["mask"])
    _, m, Sbar = sa.compress(*args, mask=dev["mask"], return_sbar=True)
    got = sa.compress_backward(*args, dS, mask=dev["mask"], sbar=Sbar, mass=m)
    torch.cuda.synchronize()
    for name, a, b in zip(("dH", "dP", "dWk", "dWv"), ref, got):
        assert torch.equal(a, b), name
    oref = sketch_batch_grad(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, dS_np, mask=inp.mask)
    tmax, tmean = TOL["bf16"]
    for name, g, r in zip(("dH", "dP", "dWk", "dWv"), got, oref):
        mx, mean = rel_errors(g.cpu().numpy(), r)
        print(f"   {name}: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert mx <= tmax and mean <= tmean, (name, mx, mean)


def test_backward_with_sbar_bench_workload_sampled():
    """40 users x 100,000 tokens, k = 1024, d = 128, the forward state from
    sa_compress_with_sbar, dS nonzero for users 5 and 31 only."""
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_config("c3lit_r40_n100k_d128_k1024")
    users = [5, 31]
    print(f"[case] backward with Sbar {inp.name} users={users}", flush=True)
    dev = upload(inp)
    args = (dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"])
    dS_np = make_sketch_grad(inp.R, inp.k, inp.d, seed=6300, users=users)
    _, m, Sbar = sa.compress(*args, mask=dev["mask"], return_sbar=True)
    del _
    dH, dP, dWk, dWv = sa.compress_backward(*args, torch.from_numpy(dS_np).to("cuda"), mask=dev["mask"],
                                            sbar=Sbar, mass=m)
    torch.cuda.synchronize()
    sel = sorted(users)
    rows = np.concatenate([np.arange(inp.offsets[u], inp.offsets[u + 1]) for u in sel])
    lens = [int(inp.offsets[u + 1] - inp.offsets[u]) for u in sel]
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    mask = None if inp.mask is None else inp.mask[rows]
    ref = sketch_batch_grad(inp.H[rows], off, inp.Wk, inp.Wv, inp.P, dS_np[sel], mask=mask)
    dH = dH.cpu().numpy()
    other = np.ones(inp.N, dtype=bool)
    other[rows] = False
    assert not dH[other].any()
    tmax, tmean = TOL["bf16"]
    for name, g, r in zip(("dH", "dP", "dWk", "dWv"), (dH[rows], dP.cpu().numpy(), dWk.cpu().numpy(),
                                                       dWv.cpu().numpy()), ref):
        mx, mean = rel_errors(g, r)
        print(f"   {name}: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert mx <= tmax and mean <= tmean, (name, mx, mean)


def test_backward_k256_d128():
    """k = 256 at d = 128: the prototype-major kernel's 8-wave shape with a
    single prototype block and 256 groups; the smoke inputs, whose last user
    (33 tokens) ends inside its first tile, so pass 1's padding slots must
    read inside H."""
    inp = make_inputs([700, 0, 2049, 33], d=128, k=256, seed=123, mask_tail_frac=0.1, name="bwd_k256_d128")
    _check(inp, make_sketch_grad(inp.R, 256, 128, seed=5256))
