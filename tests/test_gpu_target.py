"""GPU parity of sketch-branch target attention (sa_target_attention)
against the fp64 oracle on the same seeded inputs.  Bar: max_rel <= 2e-2,
mean_rel <= 2e-3 normwise over the compared outputs (fp16 sketch operands,
bf16 queries widened exactly, fp32 sums); the natural-log normalisers to an
absolute 2e-2."""
import numpy as np
import pytest

from oracle import target_attention_batch
from synth import make_candidates, make_inputs, make_sketches
from tests.gpu_util import TOL, rel_errors, upload

pytestmark = pytest.mark.gpu


def _run(Qbits, off, S):
    import torch

    import prototype_attention_compression_amd as sa
    Q = torch.from_numpy(Qbits.view(np.int16)).view(torch.bfloat16).to("cuda")
    o, lse = sa.target_attention(Q, torch.from_numpy(off).to("cuda"), torch.from_numpy(S).to("cuda"),
                                 return_lse=True)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _check(counts, k, d, seed, scale=1.0, S=None):
    Q, Qbits, off = make_candidates(counts, d, seed)
    R = len(counts)
    if S is None:
        S = make_sketches(R, k, d, seed + 1, scale)
    print(f"[case] target R={R} C={int(off[-1])} k={k} d={d} scale={scale}", flush=True)
    out, lse = _run(Qbits, off, S)
    ref, lref = target_attention_batch(Q, off, S)
    mx, mean = rel_errors(out, ref)
    lerr = float(np.abs(lse - lref).max()) if lse.size else 0.0
    print(f"   out max_rel={mx:.3e} mean_rel={mean:.3e}  lse max_abs={lerr:.3e}", flush=True)
    tmax, tmean = TOL["bf16"]
    assert np.isfinite(out).all()
    assert mx <= tmax and mean <= tmean, (mx, mean)
    assert lerr <= 2e-2
    return out


@pytest.mark.parametrize("k", [64, 320, 1024, 2048])
@pytest.mark.parametrize("d", [64, 128])
def test_target_small_ragged(k, d):
    """Users with 0, 1, 31, 33, 300 and 700 candidates: padding tiles, a
    user split over several workgroups, every k."""
    _check([0, 1, 31, 33, 300, 700], k, d, seed=6000 + k + d)


@pytest.mark.parametrize("d", [64, 128])
def test_target_largest_k(d):
    _check([300, 1, 100], 4096, d, seed=6500 + d)


@pytest.mark.parametrize("scale", [0.01, 4.0])
def test_target_flat_and_sharp(scale):
    """Nearly uniform weights (small sketch) and peaked weights (logit std 4)."""
    _check([300, 128, 5], 1024, 128, seed=6100, scale=scale)


def test_target_on_compressed_sketches():
    """End to end: the sketches sa_compress writes (zero rows for an empty
    user) feed the attention directly."""
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([3000, 0, 1200], d=128, k=512, seed=6200)
    dev = upload(inp)
    S = sa.compress(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"])
    torch.cuda.synchronize()
    out = _check([300, 300, 17], 512, 128, seed=6201, S=S.cpu().numpy())
    # the empty user's sketch is zero: every candidate gets a zero output
    assert not out[300:600].any()


def test_target_serving_workload():
    """300 users x 300 candidates against 1K x 128 sketches (the bench's
    workload), compared in full."""
    _check([300] * 300, 1024, 128, seed=6300)


def test_target_bad_offsets_zero_output():
    import torch

    import prototype_attention_compression_amd as sa
    Q, Qbits, _ = make_candidates([100, 50, 70], 128, 6400)
    S = torch.from_numpy(make_sketches(3, 256, 128, 6401)).to("cuda")
    q = torch.from_numpy(Qbits.view(np.int16)).view(torch.bfloat16).to("cuda")
    bad = torch.tensor([0, 100, 90, 220], dtype=torch.int64, device="cuda")
    o, lse = sa.target_attention(q, bad, S, return_lse=True)
    torch.cuda.synchronize()
    assert not o.any() and not lse.any()


def test_target_rows_index_a_slab():
    """sa_target_attention_rows: user u reads slab row sketch_rows[u] (rows
    repeated and out of order); equal, bit for bit, to attention over the
    gathered sketches."""
    import torch

    import prototype_attention_compression_amd as sa
    Q, Qbits, off = make_candidates([300, 0, 45, 128], 128, seed=6600)
    slab = torch.from_numpy(make_sketches(7, 512, 128, seed=6601)).to("cuda")
    rows = torch.tensor([5, 2, 5, 0], dtype=torch.int32, device="cuda")
    q = torch.from_numpy(Qbits.view(np.int16)).view(torch.bfloat16).to("cuda")
    o = torch.from_numpy(off).to("cuda")
    got = sa.target_attention(q, o, slab, sketch_rows=rows)
    want = sa.target_attention(q, o, slab[rows.long()].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref, _ = target_attention_batch(Q, off, slab[rows.long()].cpu().numpy())
    mx, mean = rel_errors(got.cpu().numpy(), ref)
    assert mx <= TOL["bf16"][0] and mean <= TOL["bf16"][1]
