"""GPU-side properties the method fixes, checked on the device output itself:
unit mass per token (sum of masses = valid tokens), closed forms (zero
prototypes -> every row is the mean value row; identical value rows -> that
row), masked == truncated, NaN in dropped rows does not propagate, empty users
give zeros, determinism, batched == per-user, token-permutation invariance,
and the device-side offsets check.  Each runs on both the one-pass and the
two-pass kernels (``path``)."""
import numpy as np
import pytest
import torch

import prototype_attention_compression_amd as sa
from oracle import sketch_batch
from synth import make_inputs
from tests.gpu_util import TOL, rel_errors, run, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(params=["one", "two"])
def path(request):
    return request.param


def _inp(lengths=(3000, 1, 4500, 0, 777), k=512, d=128, seed=31, **kw):
    return make_inputs(list(lengths), d=d, k=k, seed=seed, **kw)


def test_native_library_is_loaded():
    lib = sa.load()
    assert lib._name.endswith("prototype_attention_compression_amd/libsa.so")


def test_bitwise_deterministic(path):
    dev = upload(_inp(lengths=(40000, 9000, 31)))
    S1, m1 = run(dev, path=path)
    S2, m2 = run(dev, path=path)
    assert torch.equal(S1, S2) and torch.equal(m1, m2)


def test_total_mass_equals_valid_tokens(path):
    inp = _inp(mask_tail_frac=0.1)
    S, m = run(upload(inp), path=path)
    m = m.cpu().numpy().astype(np.float64)
    for u in range(inp.R):
        sl = inp.user_slice(u)
        n_valid = int(inp.mask[sl].sum())
        assert abs(m[u].sum() - n_valid) <= 1e-3 * max(1, n_valid), (u, m[u].sum(), n_valid)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_prototypes_give_mean_value(dtype, path):
    inp = _inp(dtype=dtype)
    inp.P[:] = 0
    if inp.P_bits is not None:
        inp.P_bits[:] = 0
    S, m = run(upload(inp), path=path)
    S = S.cpu().numpy()
    tmax, tmean = TOL[dtype]
    for u in range(inp.R):
        sl = inp.user_slice(u)
        if inp.lengths[u] == 0:
            assert not S[u].any()
            continue
        mean_v = (inp.H[sl].astype(np.float64) @ inp.Wv.astype(np.float64)).mean(axis=0)
        mx, mean = rel_errors(S[u], np.tile(mean_v, (inp.k, 1)))
        assert mx <= tmax and mean <= tmean, (u, mx, mean)
        np.testing.assert_allclose(m[u].cpu().numpy(), inp.lengths[u] / inp.k, rtol=2e-3)


def test_identical_value_rows_give_that_row(path):
    inp = _inp()
    inp.H[:, 0] = 1.0
    inp.H_bits[:, 0] = 0x3F80              # bf16 1.0
    inp.Wv[:] = 0
    inp.Wv_bits[:] = 0
    row = np.array([0.5, -2.0, 3.25, 1.0] * (inp.d // 4), dtype=np.float32)
    inp.Wv[0] = row
    from synth import f32_to_bf16_bits
    inp.Wv_bits[0] = f32_to_bf16_bits(row)
    S, _ = run(upload(inp), path=path)
    S = S.cpu().numpy()
    for u in range(inp.R):
        if inp.lengths[u]:
            np.testing.assert_allclose(S[u], np.tile(row, (inp.k, 1)), rtol=1e-5, atol=1e-6)


def test_mask_equals_truncation_and_nan_does_not_propagate(path):
    inp = _inp(mask_tail_frac=0.25)
    S_mask, m_mask = run(upload(inp), path=path)
    # NaN in every dropped row: identical result
    dev = upload(inp)
    Hn = dev["H"].clone()
    Hn[torch.from_numpy(inp.mask == 0).cuda()] = float("nan")
    dev["H"] = Hn
    S_nan, m_nan = run(dev, path=path)
    assert torch.equal(S_nan, S_mask) and torch.equal(m_nan, m_mask)
    # truncated histories: same sketches up to summation order
    keep = inp.mask == 1
    lens = [int(inp.mask[inp.user_slice(u)].sum()) for u in range(inp.R)]
    tr = make_inputs(lens, d=inp.d, k=inp.k, seed=inp.seed)
    tr.H, tr.H_bits = inp.H[keep], inp.H_bits[keep]
    tr.Wk, tr.Wk_bits, tr.Wv, tr.Wv_bits, tr.P, tr.P_bits = inp.Wk, inp.Wk_bits, inp.Wv, inp.Wv_bits, inp.P, inp.P_bits
    S_tr, m_tr = run(upload(tr), path=path)
    mx, mean = rel_errors(S_mask.cpu().numpy(), S_tr.cpu().numpy())
    assert mx <= 1e-4 and mean <= 1e-5, (mx, mean)


def test_batched_equals_single_user_calls(path):
    inp = _inp(lengths=(20000, 5, 7000, 0, 1234))
    S, m = run(upload(inp), path=path)
    S = S.cpu().numpy()
    for u in range(inp.R):
        one = make_inputs([int(inp.lengths[u])], d=inp.d, k=inp.k, seed=inp.seed)
        sl = inp.user_slice(u)
        one.H, one.H_bits = inp.H[sl], inp.H_bits[sl]
        one.Wk, one.Wk_bits, one.Wv, one.Wv_bits, one.P, one.P_bits = inp.Wk, inp.Wk_bits, inp.Wv, inp.Wv_bits, inp.P, inp.P_bits
        Su, _ = run(upload(one), path=path)
        mx, mean = rel_errors(Su.cpu().numpy()[0], S[u]) if inp.lengths[u] else (float(np.abs(S[u]).max()), 0.0)
        assert mx <= 1e-4 and mean <= 1e-5, (u, mx, mean)


def test_token_permutation_invariance(path):
    inp = _inp(lengths=(6000,))
    S, _ = run(upload(inp), path=path)
    perm = np.random.default_rng(0).permutation(inp.N)
    inp.H, inp.H_bits = inp.H[perm], inp.H_bits[perm]
    S2, _ = run(upload(inp), path=path)
    mx, mean = rel_errors(S2.cpu().numpy(), S.cpu().numpy())
    assert mx <= 1e-3 and mean <= 1e-4, (mx, mean)


def test_empty_batch_shapes(path):
    inp = _inp(lengths=(0, 0, 0))
    S, m = run(upload(inp), path=path)
    assert S.shape == (3, inp.k, inp.d) and not S.any() and not m.any()
    inp = _inp(lengths=())
    S, m = run(upload(inp), path=path)
    assert S.shape == (0, inp.k, inp.d)


def test_bad_offsets_raise_device_flag_and_zero_output(path):
    inp = _inp(lengths=(100, 200, 300))
    dev = upload(inp)
    dev["offsets"] = torch.tensor([0, 250, 200, 600], dtype=torch.int64, device="cuda")
    ws = torch.empty(sa.workspace_size(3, 600, inp.d, inp.k), dtype=torch.uint8, device="cuda")
    S, m = run(dev, workspace=ws, path=path)
    assert sa.read_device_error(ws) == 1
    assert not S.any() and not m.any()
    dev = upload(inp)
    run(dev, workspace=ws, path=path)
    assert sa.read_device_error(ws) == 0


def test_runs_on_side_stream(path):
    inp = _inp(lengths=(3000, 50))
    dev = upload(inp)
    S0, _ = run(dev, path=path)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        S1 = sa.compress(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], mask=dev["mask"], path=path)
    s.synchronize()
    assert torch.equal(S0, S1)


def test_matches_oracle_on_d64(path):
    inp = _inp(d=64, k=256, lengths=(2000, 33, 999))
    S, m = run(upload(inp), path=path)
    Sref, mref = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P)
    mx, mean = rel_errors(S.cpu().numpy(), Sref)
    assert mx <= TOL["bf16"][0] and mean <= TOL["bf16"][1]


@pytest.mark.parametrize("k", [256, 1024, 4096])
def test_one_pass_agrees_with_two_pass(k):
    """The two kernels compute the same sketches up to rounding order."""
    inp = _inp(lengths=(30000, 3, 12345, 0, 4097), k=k)
    dev = upload(inp)
    S1, m1 = run(dev, path="one")
    S2, m2 = run(dev, path="two")
    mx, mean = rel_errors(S1.cpu().numpy(), S2.cpu().numpy())
    assert mx <= 5e-3 and mean <= 5e-4, (mx, mean)
    mx, mean = rel_errors(m1.cpu().numpy(), m2.cpu().numpy())
    assert mx <= 5e-3 and mean <= 5e-4, (mx, mean)


def test_one_pass_reports_no_exchange_error():
    inp = _inp(lengths=(50000, 70000, 10))
    dev = upload(inp)
    ws = torch.empty(sa.workspace_size(inp.R, inp.N, inp.d, inp.k), dtype=torch.uint8, device="cuda")
    run(dev, workspace=ws, path="one")
    assert sa.read_device_error(ws) == 0
