"""GPU checks of the cache-miss driver: after sa_cache_lookup and
sa_cache_fill (on a side stream, the consumer waiting on an event), every
request's slab slot holds the sketch a direct sa_compress of that user alone
gives (same kernels, another batch composition: equal within fp32 summation
order, max_rel <= 1e-4), and the fp64 oracle's within the bf16 bar."""
import numpy as np
import pytest

from oracle import sketch_one
from synth import make_inputs
from tests.gpu_util import TOL, rel_errors, upload

pytestmark = pytest.mark.gpu


def test_cache_fill_matches_direct_calls():
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([0, 1, 500, 3000, 77, 4096, 33, 1200, 950, 64, 2500, 10], d=128, k=256, seed=7000,
                      mask_tail_frac=0.1)
    dev = upload(inp)
    cap = 5
    slab = torch.full((cap, 256, 128), float("nan"), device="cuda")
    mass = torch.full((cap, 256), float("nan"), device="cuda")
    cache = sa.SketchCache(cap, 256, 128, 10.0, slab, mass)
    side = torch.cuda.Stream()
    direct = {}

    def direct_sketch(u):
        if u not in direct:
            lo, hi = int(inp.offsets[u]), int(inp.offsets[u + 1])
            off = torch.tensor([0, hi - lo], dtype=torch.int64, device="cuda")
            S, m = sa.compress(dev["H"][lo:hi].contiguous(), off, dev["Wk"], dev["Wv"], dev["P"],
                               mask=dev["mask"][lo:hi].contiguous(), return_mass=True)
            direct[u] = (S[0].cpu().numpy(), m[0].cpu().numpy())
        return direct[u]

    trace = [([0, 3, 3, 7], 0.0), ([3, 8, 11, 2], 5.0), ([0, 1, 5, 3], 12.0), ([9, 10, 5, 9, 4], 13.0),
             ([2, 6], 30.0)]
    for users, now in trace:
        slots, mu, ms, st = cache.lookup(users, now)
        print(f"[case] cache batch t={now} users={users} slots={slots.tolist()} misses={mu.tolist()} {st}",
              flush=True)
        with torch.cuda.stream(side):
            cache.fill(dev["H"], inp.offsets, dev["Wk"], dev["Wv"], dev["P"], mu, ms, mask_store=dev["mask"],
                       stream=side)
            ev = torch.cuda.Event()
            ev.record(side)
        torch.cuda.current_stream().wait_event(ev)
        got = slab.cpu().numpy()
        gm = mass.cpu().numpy()
        for u, s in zip(users, slots.tolist()):
            S_d, m_d = direct_sketch(u)
            mx, _ = rel_errors(got[s], S_d)
            assert np.isfinite(got[s]).all()
            assert mx <= 1e-4, (u, s, mx)
            assert rel_errors(gm[s], m_d)[0] <= 1e-4
            lo, hi = int(inp.offsets[u]), int(inp.offsets[u + 1])
            keep = inp.mask[lo:hi] != 0
            S_ref, _ = sketch_one(inp.H[lo:hi][keep], inp.Wk, inp.Wv, inp.P)
            if np.abs(S_ref).max() > 0:
                omx, omean = rel_errors(got[s], S_ref)
                assert omx <= TOL["bf16"][0] and omean <= TOL["bf16"][1], (u, omx, omean)
            else:
                assert not got[s].any()
    # the sketch branch reads the cached sketches in place: one launch over
    # the last batch's requests through their slots
    from oracle import target_attention_batch
    from synth import make_candidates
    users, _ = trace[-1]
    slots = torch.tensor(cache.lookup(users, trace[-1][1])[0], dtype=torch.int32, device="cuda")
    Qf, Qbits, coff = make_candidates([64] * len(users), 128, seed=7001)
    q = torch.from_numpy(Qbits.view(np.int16)).view(torch.bfloat16).to("cuda")
    out = sa.target_attention(q, torch.from_numpy(coff).to("cuda"), slab, sketch_rows=slots)
    torch.cuda.synchronize()
    S_users = np.stack([direct_sketch(u)[0] for u in users])
    ref, _ = target_attention_batch(Qf, coff, S_users)
    mx, mean = rel_errors(out.cpu().numpy(), ref)
    assert mx <= TOL["bf16"][0] and mean <= TOL["bf16"][1], (mx, mean)
    cache.close()
