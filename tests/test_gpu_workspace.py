"""What pass 1 leaves in the workspace, read back after a compression whose
workspace was filled with 0xFF bytes beforehand (NaN in every float format),
so that nothing passes on a stale or lucky value.

For every tile slot of the batch (the layout restated in test_index_replay,
whose byte totals are pinned to sa_workspace_size):
  * a slot without a kept token (tile padding, masked tokens) holds a zero
    fp16 row and the -l sentinel (fp16 pair (-60000, 0));
  * a kept token's fp16 row is its bf16 row widened (exact wherever the value
    is an fp16 normal number), and its pair (hi, lo) sums to 14 - lse_t, with
    lse_t = log2 sum_j 2^(log2(e) L[j, t]) from the oracle's logits in fp64.
The sketches and masses of the same call meet the parity bar.  Covered:
both pass-1 kernels (k = 256 and 1024 keep the queries in registers, k = 320
streams them), with and without a mask."""
import numpy as np
import pytest

from oracle import logits, sketch_batch
from synth import make_inputs
from tests.gpu_util import TOL, rel_errors, upload
from tests.test_index_replay import TILE, layout, schedule, user_of

pytestmark = pytest.mark.gpu

LENGTHS = [33, 0, 1, 160, 97, 129, 31]
SENTINEL = int(np.array([-60000.0, 0.0], dtype=np.float16).view(np.uint32)[0])


@pytest.mark.parametrize("d,k,mask_frac", [(128, 1024, 0.0), (64, 256, 0.0), (128, 320, 0.0),
                                           (128, 1024, 0.25), (128, 320, 0.25)])
def test_pass1_state_in_a_poisoned_workspace(d, k, mask_frac):
    import torch

    import prototype_attention_compression_amd as sa

    inp = make_inputs(LENGTHS, d=d, k=k, seed=5100 + d + k + int(100 * mask_frac), p_scale=3.0,
                      mask_tail_frac=mask_frac, name="poisoned")
    dev = upload(inp)
    R, N = inp.R, inp.N
    L = layout(R, N, d, k, False)
    nbytes = sa.workspace_size(R, N, d, k)
    assert L["total"] == nbytes
    print(f"[case] poisoned workspace d={d} k={k} mask={mask_frac} R={R} N={N}", flush=True)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    S, m = sa.compress(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], mask=dev["mask"],
                       return_mass=True, workspace=ws)
    torch.cuda.synchronize()
    assert sa.read_device_error(ws) == 0

    Sref, mref = sketch_batch(inp.H, inp.offsets, inp.Wk, inp.Wv, inp.P, mask=inp.mask)
    S, m = S.cpu().numpy(), m.cpu().numpy()
    tmax, tmean = TOL["bf16"]
    mx, mean = rel_errors(S, Sref)
    mmx, mmean = rel_errors(m, mref)
    assert mx <= tmax and mean <= tmean, (mx, mean)
    assert mmx <= tmax and mmean <= tmean, (mmx, mmean)

    offsets, tile_base, T = schedule(LENGTHS)
    off = L["off"]
    raw = ws.cpu().numpy()
    h16 = raw[off["h16"]:off["h16"] + T * TILE * d * 2].view(np.float16).reshape(T * TILE, d)
    nl = raw[off["nl"]:off["nl"] + T * TILE * 4].view(np.uint32)
    pair = nl.view(np.float16).reshape(-1, 2).astype(np.float64)

    t = np.arange(T)
    u = user_of(tile_base, t)
    tok = (offsets[u][:, None] + (t - tile_base[u])[:, None] * TILE + np.arange(TILE)[None, :]).reshape(-1)
    end = np.repeat(offsets[u + 1], TILE)
    kept = tok < end
    if inp.mask is not None:
        kept &= inp.mask[np.minimum(tok, N - 1)] != 0
    assert (~kept).any() and kept.any()

    # dropped slots: zero rows (every bit) and the sentinel
    assert not h16[~kept].view(np.uint16).any()
    assert np.all(nl[~kept] == SENTINEL)

    # kept slots: the widened row, and 14 - lse
    Hk = inp.H[tok[kept]].astype(np.float32)
    got = h16[kept].astype(np.float32)
    normal = np.abs(Hk) >= 2.0 ** -14
    assert np.array_equal(got[normal], Hk[normal])
    assert np.all(np.abs(got[~normal] - Hk[~normal]) < 2.0 ** -24)
    lse = np.empty(N)
    for uu in range(R):
        a, b = int(inp.offsets[uu]), int(inp.offsets[uu + 1])
        if b > a:
            Lg = logits(inp.H[a:b], inp.Wk, inp.P)                # [k, n], natural units
            c = Lg.max(axis=0)
            lse[a:b] = (c + np.log(np.exp(Lg - c).sum(axis=0))) / np.log(2.0)
    want = 14.0 - lse[tok[kept]]
    err = np.abs(pair[kept].sum(axis=1) - want)
    spread = np.ptp(want)
    print(f"   S max_rel={mx:.2e}  -l max err={err.max():.2e} (spread of -l over tokens {spread:.2f})", flush=True)
    # (measured 0.8e-5 - 2.6e-5: fp16 operands, fp32 sums; a misplaced token
    # would be off by up to the spread, 0.1 - 0.3 here)
    assert err.max() < 1e-3 < spread
