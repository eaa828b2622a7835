"""GPU parity: libsa (HIP, gfx950) against the fp64 oracle on the same seeded
inputs.  Bar: bf16 inputs max_rel <= 2e-2 and mean_rel <= 2e-3, fp32 inputs
<= 1e-4 (normwise over all compared sketch elements); masses to the same
bar.  Full-size workloads compare a sample of users (the oracle computes one
user at a time) in the very launch configuration the bench times (the
library's own path choice), and again with each path forced: "one" (the
one-pass kernel with the cross-workgroup exchange; for shapes it is not built
for the library runs two passes) and "two" (two passes)."""
import numpy as np
import pytest

from oracle import sketch_batch
from synth import make_config
from tests.gpu_util import TOL, rel_errors, run, upload

pytestmark = pytest.mark.gpu

SMALL = ["c1_fp32_n4096_d64_k64", "small_ragged_d128_k256", "small_ragged_d128_k1024",
         "small_ragged_d64_k128", "small_mask_d128_k512", "small_fp32_ragged_d128_k192"]


def _check(inp, users=None, path=None):
    dev = upload(inp)
    print(f"[case] {inp.name} R={inp.R} N={inp.N} k={inp.k} d={inp.d} dtype={inp.dtype} users={users} "
          f"path={path}", flush=True)
    S, m = run(dev, path=path)
    S = S.cpu().numpy()
    m = m.cpu().numpy()
    Sref, mref = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask, users=users)
    sel = list(range(inp.R)) if users is None else list(users)
    mx, mean = rel_errors(S[sel], Sref[sel])
    mmx, mmean = rel_errors(m[sel], mref[sel])
    tmax, tmean = TOL[inp.dtype]
    print(f"   S max_rel={mx:.3e} mean_rel={mean:.3e}  mass max_rel={mmx:.3e} mean_rel={mmean:.3e}", flush=True)
    assert np.isfinite(S).all() and np.isfinite(m).all()
    assert mx <= tmax and mean <= tmean, (mx, mean)
    assert mmx <= tmax and mmean <= tmean, (mmx, mmean)
    # users outside the sample must still be finite, and empty users exactly zero
    for u in range(inp.R):
        if inp.lengths[u] == 0:
            assert not S[u].any() and not m[u].any()
    return S, m


@pytest.mark.parametrize("path", ["one", "two"])
@pytest.mark.parametrize("name", SMALL)
def test_parity_small(name, path):
    _check(make_config(name), path=path)


@pytest.mark.parametrize("k", [256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("d", [64, 128])
def test_parity_one_pass_every_block_count(k, d):
    """Every built prototype-block count (k / 256 = 1 .. 16 workgroups per
    group), ragged users with empty, one-token and tile-straddling lengths."""
    from synth import make_inputs
    inp = make_inputs([2049, 0, 1, 5000, 31, 700], d=d, k=k, seed=1000 + k + d)
    _check(inp, path="one")


@pytest.mark.parametrize("k", [64, 320, 1024, 2048])
@pytest.mark.parametrize("d", [64, 128])
def test_parity_many_short_users(k, d):
    """Pass 2's groups walk equal tile ranges cut at user boundaries: with 200
    short ragged users (some empty) every group crosses many users, and each
    user's sums come from several groups' partial slots.  k = 64 .. 2048
    covers 1 .. 8 prototype blocks per group (k = 320: five blocks, a group
    count that is not a multiple of 8)."""
    from synth import make_inputs
    rng = np.random.default_rng(2000 + k + d)
    lens = rng.integers(0, 400, size=200)
    lens[::17] = 0
    inp = make_inputs(lens.tolist(), d=d, k=k, seed=3000 + k + d)
    _check(inp, path="two")


@pytest.mark.parametrize("R", [2047, 2048, 2049, 6000])
def test_parity_thousands_of_users(R):
    """The schedule takes users 2048 at a time (8 per thread, a running carry
    between the passes): user counts on both sides of a pass boundary and
    several passes, short ragged users (a fifth of them empty), every
    sketch and mass compared with the oracle."""
    from synth import make_inputs
    rng = np.random.default_rng(2400 + R)
    lens = rng.integers(0, 48, size=R)
    lens[rng.random(R) < 0.2] = 0
    inp = make_inputs(lens.tolist(), d=64, k=64, seed=3400 + R, name=f"users{R}")
    _check(inp, path="two")


def _sample(inp, n_random=2, seed=0):
    lens = inp.lengths
    pick = {int(np.argmin(lens)), int(np.argmax(lens))}
    rng = np.random.default_rng(seed)
    while len(pick) < min(inp.R, 2 + n_random):
        pick.add(int(rng.integers(0, inp.R)))
    return sorted(pick)


@pytest.mark.parametrize("path", [None, "two"])
def test_parity_c2_single_user_100k(path):
    _check(make_config("c2_n100k_d128_k1024"), path=path)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_parity_few_long_users_presummed(dtype):
    """Few users, one of them long: its many partial slots are pre-summed in
    sub-ranges before the finalize (the fp32 path's chunks and the bf16
    path's group slots), next to short users that are not."""
    from synth import make_inputs
    inp = make_inputs([20000, 3, 0, 1500], d=64, k=128, seed=1400, dtype=dtype, name=f"presum_{dtype}")
    _check(inp, path="two")


def test_parity_bench_workload_sampled():
    """40 users x 100,000 tokens, k = 1024, d = 128: the bench's workload and
    launch configuration."""
    inp = make_config("c3lit_r40_n100k_d128_k1024")
    _check(inp, users=[0, 17, 39])


def test_parity_c3_training_batch_sampled():
    inp = make_config("c3_r40_ragged_d128_k1024")
    _check(inp, users=_sample(inp))


def test_parity_c4_serving_batch_sampled():
    inp = make_config("c4_r120_lognormal_d128_k1024")
    _check(inp, users=_sample(inp, n_random=1))


@pytest.mark.parametrize("name", ["c5_r8_n100k_d128_k256", "c5_r8_n100k_d128_k512",
                                  "c5_r8_n100k_d128_k2048", "c5mask_r8_n100k_d128_k1024"])
def test_parity_c5_sweep_sampled(name):
    inp = make_config(name)
    _check(inp, users=[0, inp.R - 1])


@pytest.mark.parametrize("path", [None, "two"])
def test_parity_sharp_softmax(path):
    """Peaked softmax (logit std about 4): both paths take their exact,
    max-shifted exponent mode here."""
    _check(make_config("sharp_n100k_d128_k1024"), path=path)


def test_parity_clustered_history():
    inp = make_config("clustered_r4_n100k_d128_k1024")
    _check(inp, users=[1, 3])
