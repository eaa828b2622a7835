"""GPU parity at the method's edge cases, against the fp64 oracles.

* The hard-assignment limit of the per-token softmax over prototypes, with
  prototypes that receive no mass although tokens are present (blog "100,000
  videos in your pocket", "How it works" item 1: every item distributes its
  mass over the prototypes; a prototype no item reaches has zero mass, and
  the zero-mass reading gives it a zero row).  Logits reach about 1,500 (base
  2), so both pass 1's max-shifted mode and the fp16 underflow of the
  allocations run; every non-winning logit trails its token's winners by more
  than 745, so the oracle's zero masses are exact zeros too, and the GPU
  must reproduce them exactly.
* Range errors: a kept bf16 history value outside fp16's finite range (the
  MFMA operand type) raises a device error bit; masked values never do.
* Target attention over a sketch array indexed by row: an index outside the
  array reads nothing, zeroes that user's outputs and raises a bit.
Bar: bf16 max_rel <= 2e-2, mean_rel <= 2e-3 (normwise)."""
import numpy as np
import pytest

from oracle import logits, sketch_batch, sketch_batch_grad, target_attention_batch
from synth import (f32_to_bf16_bits, make_candidates, make_hard_assignment_inputs, make_inputs,
                   make_sketch_grad, make_sketches)
from tests.gpu_util import TOL, rel_errors, run, upload

pytestmark = pytest.mark.gpu


def _winner_gap(inp):
    """Smallest distance between a token's top logit and its first logit
    more than 760 below it (the construction's precondition)."""
    L = logits(inp.H, inp.Wk, inp.P)
    top = L.max(axis=0, keepdims=True)
    far = np.where(L >= top - 760, -np.inf, L).max(axis=0)
    return float((top[0] - far).min())


@pytest.mark.parametrize("path", [None, "one"])
@pytest.mark.parametrize("d,k", [(64, 64), (128, 256), (128, 1024)])
def test_hard_assignment_forward(d, k, path):
    inp = make_hard_assignment_inputs([700, 0, 2049, 33, 5000], d=d, k=k, seed=7000 + d + k, name=f"hard_d{d}_k{k}")
    assert _winner_gap(inp) > 745.0
    print(f"[case] hard assignment R={inp.R} N={inp.N} k={k} d={d} path={path}", flush=True)
    dev = upload(inp)
    S, m = run(dev, path=path)
    S, m = S.cpu().numpy(), m.cpu().numpy()
    Sref, mref = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P)
    mx, mean = rel_errors(S, Sref)
    mmx, mmean = rel_errors(m, mref)
    zero = mref == 0.0
    print(f"   S max_rel={mx:.3e} mean_rel={mean:.3e}  mass max_rel={mmx:.3e} mean_rel={mmean:.3e}  "
          f"zero-mass prototypes {int(zero.sum())} of {zero.size}", flush=True)
    tmax, tmean = TOL["bf16"]
    assert np.isfinite(S).all() and np.isfinite(m).all()
    assert mx <= tmax and mean <= tmean
    assert mmx <= tmax and mmean <= tmean
    # prototypes no token reaches, in users that have tokens: exact zeros
    assert zero[0].any() and not zero[0].all()
    assert (m[zero] == 0.0).all(), "zero-mass prototypes get exactly zero mass"
    assert not S[zero].any(), "zero-mass prototypes get exactly zero rows"
    # masses of prototypes that only hard tokens reach are whole counts
    assert np.abs(m[~zero] - mref[~zero]).max() <= 1e-3 * max(1.0, np.abs(mref).max())


@pytest.mark.parametrize("d,k", [(64, 64), (128, 512)])
def test_hard_assignment_backward(d, k):
    """At a saturated softmax the Jacobian of the allocations vanishes for the
    hard tokens; the soft tokens (two winners) keep dP and dWk nonzero.
    Zero-mass rows pass no gradient."""
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_hard_assignment_inputs([700, 0, 2049, 33], d=d, k=k, seed=7100 + d + k, name=f"hard_bwd_d{d}_k{k}")
    assert _winner_gap(inp) > 745.0
    print(f"[case] hard assignment backward R={inp.R} N={inp.N} k={k} d={d}", flush=True)
    dev = upload(inp)
    dS = make_sketch_grad(inp.R, k, d, seed=7200 + d)
    out = sa.compress_backward(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"],
                               torch.from_numpy(dS).to("cuda"))
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in out]
    ref = sketch_batch_grad(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, dS)
    tmax, tmean = TOL["bf16"]
    for name, g, r in zip(("dH", "dP", "dWk", "dWv"), got, ref):
        mx, mean = rel_errors(g, r)
        print(f"   {name}: max_rel={mx:.3e} mean_rel={mean:.3e}", flush=True)
        assert np.isfinite(g).all(), name
        assert mx <= tmax and mean <= tmean, (name, mx, mean)


# ---------------------------------------------------------------- range errors
def _bf16_tensor(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def _bf16_bits_of(value: float) -> int:
    if np.isnan(value):
        return 0x7FC0
    if np.isinf(value):
        return 0x7F80 if value > 0 else 0xFF80
    return int(f32_to_bf16_bits(np.array([value], dtype=np.float32))[0])


@pytest.mark.parametrize("k,path", [(1024, None), (320, None), (256, "one")])
def test_range_flag_forward(k, path):
    """A kept history value outside fp16's range (70144, inf, NaN) raises
    SA_DEVICE_ERR_RANGE in every pass-1 form (k = 1024: queries in
    registers; k = 320: queries streamed; the one-pass packing kernel); the
    same value in a masked row does not, and the next clean call on the
    workspace clears the flag."""
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([300, 0, 1000], d=128, k=k, seed=7300 + k, mask_tail_frac=0.2)
    dev = upload(inp)
    ws = torch.empty(sa.workspace_size(inp.R, inp.N, 128, k), dtype=torch.uint8, device="cuda")
    args = lambda H: (H, dev["offsets"], dev["Wk"], dev["Wv"], dev["P"])  # noqa: E731
    kept = int(inp.offsets[2]) + 17           # a kept token of user 2
    dropped = int(inp.offsets[3]) - 1         # the last token of user 2 is masked
    assert inp.mask[kept] == 1 and inp.mask[dropped] == 0
    for value in (70000.0, np.inf, np.nan, -1.0e6):
        print(f"[case] range flag k={k} path={path} value={value}", flush=True)
        bits = inp.H_bits.copy()
        bits[kept, 5] = _bf16_bits_of(value)
        sa.compress(*args(_bf16_tensor(bits)), mask=dev["mask"], workspace=ws, path=path)
        assert sa.read_device_error(ws) & sa.SA_DEVICE_ERR_RANGE
        bits = inp.H_bits.copy()
        bits[dropped, 3] = 0x7FC0                  # NaN in a masked row
        bits[dropped, 4] = _bf16_bits_of(1.0e6)
        S = sa.compress(*args(_bf16_tensor(bits)), mask=dev["mask"], workspace=ws, path=path)
        assert sa.read_device_error(ws) == 0
        assert torch.isfinite(S).all()
    # 65280, the largest bf16 value not above 65504, is in range
    bits = inp.H_bits.copy()
    bits[kept, 5] = _bf16_bits_of(65280.0)
    sa.compress(*args(_bf16_tensor(bits)), mask=dev["mask"], workspace=ws, path=path)
    assert sa.read_device_error(ws) == 0


def test_range_flag_backward():
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([300, 1000], d=128, k=512, seed=7400)
    dev = upload(inp)
    bits = inp.H_bits.copy()
    bits[400, 9] = 0x7F80                           # +inf in a kept row
    ws = torch.empty(sa.backward_workspace_size(inp.R, inp.N, 128, 512), dtype=torch.uint8, device="cuda")
    dS = torch.from_numpy(make_sketch_grad(inp.R, 512, 128, seed=7401)).to("cuda")
    sa.compress_backward(_bf16_tensor(bits), dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], dS, workspace=ws)
    assert sa.read_device_error(ws) & sa.SA_DEVICE_ERR_RANGE


# ---------------------------------------------------------------- target attention edges
def test_target_rows_out_of_range_reads_nothing():
    """Users whose sketch_rows index falls outside the slab get zero outputs
    and raise SA_DEVICE_ERR_SKETCH_ROW; the other users' outputs equal the
    in-range call's bit for bit."""
    import torch

    import prototype_attention_compression_amd as sa
    Q, Qbits, off = make_candidates([300, 40, 45, 128, 7], 128, seed=7500)
    slab = torch.from_numpy(make_sketches(6, 1024, 128, seed=7501)).to("cuda")
    q = _bf16_tensor(Qbits)
    o = torch.from_numpy(off).to("cuda")
    ws = torch.empty(sa.target_attention_workspace_size(5, int(off[-1]), 128, 1024), dtype=torch.uint8,
                     device="cuda")
    good = torch.tensor([5, 2, 3, 0, 1], dtype=torch.int32, device="cuda")
    bad = torch.tensor([5, 6, -1, 0, 1 << 30], dtype=torch.int32, device="cuda")
    want, lse_w = sa.target_attention(q, o, slab, sketch_rows=good, return_lse=True, workspace=ws)
    assert sa.read_device_error(ws) == 0
    got, lse_g = sa.target_attention(q, o, slab, sketch_rows=bad, return_lse=True, workspace=ws)
    assert sa.read_device_error(ws) & sa.SA_DEVICE_ERR_SKETCH_ROW
    torch.cuda.synchronize()
    for u in range(5):
        sl = slice(int(off[u]), int(off[u + 1]))
        if u in (1, 2, 4):
            assert not got[sl].any() and not lse_g[sl].any()
        else:
            assert torch.equal(got[sl], want[sl]) and torch.equal(lse_g[sl], lse_w[sl])
    ref, _ = target_attention_batch(Q, off, slab[good.long()].cpu().numpy())
    mx, mean = rel_errors(want.cpu().numpy(), ref)
    assert mx <= TOL["bf16"][0] and mean <= TOL["bf16"][1]


def test_target_range_flag():
    import torch

    import prototype_attention_compression_amd as sa
    Q, Qbits, off = make_candidates([100, 33], 128, seed=7600)
    S = torch.from_numpy(make_sketches(2, 256, 128, seed=7601)).to("cuda")
    o = torch.from_numpy(off).to("cuda")
    ws = torch.empty(sa.target_attention_workspace_size(2, int(off[-1]), 128, 256), dtype=torch.uint8,
                     device="cuda")
    sa.target_attention(_bf16_tensor(Qbits), o, S, workspace=ws)
    assert sa.read_device_error(ws) == 0
    bits = Qbits.copy()
    bits[120, 7] = 0xFF80                          # -inf query value
    sa.target_attention(_bf16_tensor(bits), o, S, workspace=ws)
    assert sa.read_device_error(ws) & sa.SA_DEVICE_ERR_RANGE
    S2 = S.clone()
    S2[1, 17, 3] = 1.0e5                           # sketch value beyond fp16
    sa.target_attention(_bf16_tensor(Qbits), o, S2, workspace=ws)
    assert sa.read_device_error(ws) & sa.SA_DEVICE_ERR_RANGE
