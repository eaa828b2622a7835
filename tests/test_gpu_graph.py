"""sa_compress captured in a HIP graph (through torch.cuda.graph) replays to
the eager result bit for bit.  The launch sequence holds no memset and
allocates nothing, so it can be captured.  Each replay is checked, with eager
calls and synchronisations between the replays, after the outputs were
overwritten outside the graph."""
import numpy as np
import pytest

from synth import make_inputs
from tests.gpu_util import upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,k", [(128, 1024), (64, 256)])
def test_graph_replays_equal_eager(d, k):
    import torch

    import prototype_attention_compression_amd as sa
    inp = make_inputs([700, 0, 2049, 33, 1], d=d, k=k, seed=6100 + k, mask_tail_frac=0.1, name=f"graph_k{k}")
    print(f"[case] graph capture R={inp.R} N={inp.N} k={k} d={d}", flush=True)
    dev = upload(inp)
    R, N = inp.R, inp.N
    ws = torch.empty(sa.workspace_size(R, N, d, k), dtype=torch.uint8, device="cuda")
    S = torch.empty((R, k, d), dtype=torch.float32, device="cuda")
    m = torch.empty((R, k), dtype=torch.float32, device="cuda")

    def step():
        sa.compress(dev["H"], dev["offsets"], dev["Wk"], dev["Wv"], dev["P"], mask=dev["mask"],
                    return_mass=True, out=S, mass_out=m, workspace=ws)

    step()
    torch.cuda.synchronize()
    S_ref, m_ref = S.clone(), m.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        S.fill_(np.nan)
        m.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, S_ref) and torch.equal(m, m_ref), f"replay {r}"
        step()   # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(S, S_ref)
