"""The MFMA rate probe (sa_probe_mfma) does the work it reports.

With the constant operands (every fp16 value 1/64) each 32x32x16 MFMA adds
16 / 4096 to every accumulator element; a wave runs 2 MFMAs per chain and
iteration, so each thread's sum over its 4 chains x 16 elements is exactly
iters / 2 (powers of two: no rounding).  Zero operands give exactly 0."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters", [1, 10, 4096])
def test_probe_sink_values(iters):
    import torch

    from prototype_attention_compression_amd import _lib
    sink = torch.full((_lib.PROBE_SINK_FLOATS,), -1.0, dtype=torch.float32, device="cuda")
    print(f"[case] probe iters={iters}", flush=True)
    flop = _lib.probe_mfma(1, iters, sink)
    torch.cuda.synchronize()
    assert flop == 2048.0 * iters * 8 * 32768
    assert torch.equal(sink, torch.full_like(sink, iters / 2.0))
    _lib.probe_mfma(0, iters, sink)
    torch.cuda.synchronize()
    assert not sink.any()
    _lib.probe_mfma(2, iters, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all() and sink.abs().sum() > 0
