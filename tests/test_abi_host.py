"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/sa.h declares, and rejects bad arguments before any
HIP call."""
import ctypes
import os
import re

import pytest

import prototype_attention_compression_amd as sa
from prototype_attention_compression_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "sa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_]+)\s*\(", src)))


def test_header_declarations_are_exported():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert re.fullmatch(r"\d+\.\d+\.\d+", sa.version())
    for s in range(5):
        assert sa.status_string(s).startswith("SA_")
    assert sa.status_string(99) == "unknown sa_status"


def _ws(R, N, d, k, dt, flags=0):
    pb = _lib.SaProblem(R, N, d, k, dt, flags)
    out = ctypes.c_size_t(0)
    st = _lib.load().sa_workspace_size(ctypes.byref(pb), ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("args,code", [
    ((-1, 10, 128, 1024, 0), sa.SA_E_INVALID),
    ((1, -10, 128, 1024, 0), sa.SA_E_INVALID),
    ((1, 10, 0, 1024, 0), sa.SA_E_INVALID),
    ((1, 10, 128, 0, 0), sa.SA_E_INVALID),
    ((1, 10, 128, 1024, 7), sa.SA_E_INVALID),
    ((1, 10, 96, 1024, 0), sa.SA_E_UNSUPPORTED),
    ((1, 10, 128, 1000, 0), sa.SA_E_UNSUPPORTED),
    ((1, 10, 128, 8192, 0), sa.SA_E_UNSUPPORTED),
    ((1, 1 << 31, 128, 1024, 0), sa.SA_E_UNSUPPORTED),
])
def test_workspace_size_rejects(args, code):
    assert _ws(*args)[0] == code


def test_workspace_size_flags_and_null():
    assert _ws(1, 10, 128, 1024, 0, flags=4)[0] == sa.SA_E_INVALID
    assert _ws(1, 10, 128, 1024, 0, flags=sa.SA_FLAG_ONE_PASS | sa.SA_FLAG_TWO_PASS)[0] == sa.SA_E_INVALID
    base = _ws(1, 10, 128, 1024, 0)
    assert base[0] == sa.SA_OK
    for f in (sa.SA_FLAG_ONE_PASS, sa.SA_FLAG_TWO_PASS):
        assert _ws(1, 10, 128, 1024, 0, flags=f) == base   # one workspace serves both paths
    pb = _lib.problem(1, 10, 128, 1024, 0)
    assert _lib.load().sa_workspace_size(ctypes.byref(pb), None) == sa.SA_E_INVALID
    assert _lib.load().sa_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == sa.SA_E_INVALID


def test_workspace_size_grows():
    base = sa.workspace_size(4, 10_000, 128, 1024)
    assert sa.workspace_size(4, 20_000, 128, 1024) > base
    assert sa.workspace_size(8, 10_000, 128, 1024) > base
    assert sa.workspace_size(4, 10_000, 128, 2048) > base
    assert sa.workspace_size(0, 0, 64, 64) > 0
    for dt in (sa.SA_BF16, sa.SA_F32):
        assert sa.workspace_size(3, 1000, 64, 128, dt) % 256 == 0


FAKE = 0x100000  # never dereferenced: every case below fails before any HIP call


def _call(pb, H=FAKE, off=FAKE, mask=None, Wk=FAKE, Wv=FAKE, P=FAKE, S=FAKE, mass=None,
          ws=FAKE, wsb=1 << 40):
    return _lib.raw_compress(pb, H, off, mask, Wk, Wv, P, S, mass, ws, wsb, None)


def test_compress_argument_errors_before_launch():
    lib = _lib.load()
    vp = None
    assert lib.sa_compress(None, vp, vp, vp, vp, vp, vp, vp, vp, vp, 0, vp) == sa.SA_E_INVALID
    pb = _lib.problem(2, 100, 128, 256, 0)
    assert _call(pb, off=None) == sa.SA_E_INVALID
    assert _call(pb, H=None) == sa.SA_E_INVALID
    assert _call(pb, Wk=None) == sa.SA_E_INVALID
    assert _call(pb, Wv=None) == sa.SA_E_INVALID
    assert _call(pb, P=None) == sa.SA_E_INVALID
    assert _call(pb, S=None) == sa.SA_E_INVALID
    assert _call(pb, ws=None) == sa.SA_E_WORKSPACE
    need = sa.workspace_size(2, 100, 128, 256)
    assert _call(pb, wsb=need - 1) == sa.SA_E_WORKSPACE
    assert _call(pb, ws=FAKE + 16, wsb=need) == sa.SA_E_INVALID        # misaligned
    assert _call(_lib.problem(2, 100, 96, 256, 0)) == sa.SA_E_UNSUPPORTED
    assert _call(_lib.problem(-2, 100, 128, 256, 0)) == sa.SA_E_INVALID


def test_zero_users_is_a_noop():
    # R = 0 returns before touching any pointer or the GPU
    pb = _lib.problem(0, 0, 128, 1024, 0)
    assert _call(pb, H=None, off=None, Wk=None, Wv=None, P=None, S=None, ws=None, wsb=0) == sa.SA_OK


def test_binding_validates_before_library():
    import torch
    H = torch.zeros(4, 128, dtype=torch.bfloat16)
    off = torch.tensor([0, 4])
    with pytest.raises(ValueError):
        sa.compress(H, off, H[:0], H[:0], H[:0])   # CPU tensors are refused


# ---------------------------------------------------------------- backward
def _bws(R, N, d, k, dt, flags=0):
    pb = _lib.SaProblem(R, N, d, k, dt, flags)
    out = ctypes.c_size_t(0)
    st = _lib.load().sa_backward_workspace_size(ctypes.byref(pb), ctypes.byref(out))
    return st, out.value


def test_backward_workspace_size():
    assert _bws(2, 1000, 128, 1024, sa.SA_BF16)[0] == sa.SA_OK
    assert _bws(2, 1000, 128, 1024, sa.SA_F32)[0] == sa.SA_E_UNSUPPORTED
    assert _bws(2, 1000, 128, 1024, sa.SA_BF16, sa.SA_FLAG_ONE_PASS)[0] == sa.SA_E_UNSUPPORTED
    assert _bws(2, 1000, 128, 1024, sa.SA_BF16, sa.SA_FLAG_TWO_PASS)[0] == sa.SA_OK
    assert _bws(2, 1000, 96, 1024, sa.SA_BF16)[0] == sa.SA_E_UNSUPPORTED
    assert _bws(2, 1000, 128, 1000, sa.SA_BF16)[0] == sa.SA_E_UNSUPPORTED
    # the backward needs the forward's buffers and more
    for R, N, d, k in ((2, 1000, 128, 1024), (40, 4_000_000, 128, 1024), (3, 77, 64, 320)):
        st, b = _bws(R, N, d, k, sa.SA_BF16)
        assert st == sa.SA_OK and b % 256 == 0
        assert b > sa.workspace_size(R, N, d, k)
    pb = _lib.problem(1, 10, 128, 1024, 0)
    assert _lib.load().sa_backward_workspace_size(ctypes.byref(pb), None) == sa.SA_E_INVALID


def _bcall(pb, H=FAKE, off=FAKE, mask=None, Wk=FAKE, Wv=FAKE, P=FAKE, dS=FAKE, dH=FAKE, dP=FAKE, dWk=FAKE,
           dWv=FAKE, ws=FAKE, wsb=1 << 40):
    return _lib.raw_compress_backward(pb, H, off, mask, Wk, Wv, P, dS, dH, dP, dWk, dWv, ws, wsb, None)


def test_backward_argument_errors_before_launch():
    lib = _lib.load()
    vp = None
    assert lib.sa_compress_backward(None, *([vp] * 12), 0, vp) == sa.SA_E_INVALID
    pb = _lib.problem(2, 100, 128, 512, 0)
    for name in ("off", "H", "Wk", "Wv", "P", "dS", "dH", "dP", "dWk", "dWv"):
        assert _bcall(pb, **{name: None}) == sa.SA_E_INVALID, name
    assert _bcall(pb, ws=None) == sa.SA_E_WORKSPACE
    need = _bws(2, 100, 128, 512, 0)[1]
    assert _bcall(pb, wsb=need - 1) == sa.SA_E_WORKSPACE
    assert _bcall(pb, ws=FAKE + 16, wsb=need) == sa.SA_E_INVALID
    assert _bcall(_lib.problem(2, 100, 128, 512, sa.SA_F32)) == sa.SA_E_UNSUPPORTED
    assert _bcall(_lib.problem(2, 100, 128, 512, 0, sa.SA_FLAG_ONE_PASS)) == sa.SA_E_UNSUPPORTED
    # no tokens: H and dH may be NULL (the call would then launch, so only
    # the argument checks that come first are exercised here)
    assert _bcall(_lib.problem(2, 0, 128, 512, 0), H=None, dH=None, ws=None) == sa.SA_E_WORKSPACE


def test_backward_binding_validates_before_library():
    import torch
    H = torch.zeros(4, 128, dtype=torch.bfloat16)
    off = torch.tensor([0, 4])
    with pytest.raises(ValueError):
        sa.compress_backward(H, off, H[:0], H[:0], H[:0], torch.zeros(1, 1, 128))
    with pytest.raises(ValueError):
        sa.compress_backward(H.float(), off, H[:0], H[:0], H[:0], torch.zeros(1, 1, 128))


# ---------------------------------------------------------------- target attention
def test_target_attention_argument_errors_before_launch():
    lib = _lib.load()
    out = ctypes.c_size_t(0)
    pb = _lib.problem(3, 900, 128, 1024, sa.SA_BF16)
    assert lib.sa_target_attention_workspace_size(ctypes.byref(pb), ctypes.byref(out)) == sa.SA_OK
    need = out.value
    assert need % 256 == 0 and need > 0
    for bad in (_lib.problem(3, 900, 128, 1024, sa.SA_F32), _lib.problem(3, 900, 128, 1024, 0, 1),
                _lib.problem(3, 900, 96, 1024, 0)):
        assert lib.sa_target_attention_workspace_size(ctypes.byref(bad), ctypes.byref(out)) == sa.SA_E_UNSUPPORTED

    def call(pb, Q=FAKE, off=FAKE, S=FAKE, o=FAKE, lse=None, ws=FAKE, wsb=1 << 40):
        return _lib.raw_target_attention(pb, Q, off, S, o, lse, ws, wsb, None)

    assert call(pb, off=None) == sa.SA_E_INVALID
    assert call(pb, S=None) == sa.SA_E_INVALID
    assert call(pb, Q=None) == sa.SA_E_INVALID
    assert call(pb, o=None) == sa.SA_E_INVALID
    assert call(pb, S=FAKE + 4) == sa.SA_E_INVALID          # misaligned sketch
    assert call(pb, ws=None) == sa.SA_E_WORKSPACE
    assert call(pb, wsb=need - 1) == sa.SA_E_WORKSPACE
    assert call(_lib.problem(0, 0, 128, 1024, 0), Q=None, off=None, S=None, o=None, ws=None, wsb=0) == sa.SA_OK
    # the row-indexed form: a negative sketch count is an argument error
    rows = FAKE + 256
    assert _lib.raw_target_attention(pb, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None, sketch_rows=rows,
                                     sketch_count=-1) == sa.SA_E_INVALID
    assert _lib.raw_target_attention(pb, FAKE, FAKE, FAKE, FAKE, None, None, 0, None, sketch_rows=rows,
                                     sketch_count=7) == sa.SA_E_WORKSPACE
    assert lib.sa_target_attention(None, *([None] * 6), 0, None) == sa.SA_E_INVALID


def test_workspace_bytes_matches_workspace_size():
    lib = _lib.load()
    for R, N, d, k, dt in ((1, 100_000, 128, 1024, 0), (40, 4_000_000, 128, 1024, 0), (3, 77, 64, 320, 1),
                           (0, 0, 128, 256, 0)):
        pb = _lib.problem(R, N, d, k, dt)
        assert lib.sa_workspace_bytes(ctypes.byref(pb)) == sa.workspace_size(R, N, d, k, dt)
    assert lib.sa_workspace_bytes(None) == 0
    bad = _lib.problem(1, 10, 96, 1024, 0)
    assert lib.sa_workspace_bytes(ctypes.byref(bad)) == 0


def test_unknown_flag_bits_are_invalid():
    for bit in (4, 8, 1 << 30):
        assert _ws(1, 10, 128, 1024, 0, flags=bit)[0] == sa.SA_E_INVALID
        assert _bws(1, 10, 128, 1024, 0, flags=bit)[0] == sa.SA_E_INVALID




# ---------------------------------------------------------------- forward state for the backward
def test_compress_with_sbar_argument_errors_before_launch():
    pb = _lib.problem(2, 100, 128, 256, 0)

    def call(pb, mass=FAKE, Sbar=FAKE, ws=FAKE, wsb=1 << 40, S=FAKE):
        return _lib.raw_compress_with_sbar(pb, FAKE, FAKE, None, FAKE, FAKE, FAKE, S, mass, Sbar, ws, wsb, None)

    assert call(pb, mass=None) == sa.SA_E_INVALID
    assert call(pb, Sbar=None) == sa.SA_E_INVALID
    assert call(pb, S=None) == sa.SA_E_INVALID
    assert call(pb, ws=None) == sa.SA_E_WORKSPACE
    assert call(_lib.problem(2, 100, 96, 256, 0)) == sa.SA_E_UNSUPPORTED
    # R = 0 is a no-op whatever the pointers
    assert call(_lib.problem(0, 0, 128, 256, 0), mass=None, Sbar=None, S=None, ws=None, wsb=0) == sa.SA_OK
    assert _lib.load().sa_compress_with_sbar(None, *([None] * 10), 0, None, None) == sa.SA_E_INVALID


def test_backward_with_sbar_argument_errors_before_launch():
    pb = _lib.problem(2, 100, 128, 512, 0)

    def call(pb, Sbar=FAKE, mass=FAKE, ws=FAKE, wsb=1 << 40, **kw):
        a = dict(H=FAKE, off=FAKE, Wk=FAKE, Wv=FAKE, P=FAKE, dS=FAKE, dH=FAKE, dP=FAKE, dWk=FAKE, dWv=FAKE)
        a.update(kw)
        return _lib.raw_compress_backward_with_sbar(pb, a["H"], a["off"], None, a["Wk"], a["Wv"], a["P"], Sbar,
                                                    mass, a["dS"], a["dH"], a["dP"], a["dWk"], a["dWv"], ws, wsb,
                                                    None)

    assert call(pb, Sbar=None) == sa.SA_E_INVALID
    assert call(pb, mass=None) == sa.SA_E_INVALID
    for name in ("off", "H", "Wk", "Wv", "P", "dS", "dH", "dP", "dWk", "dWv"):
        assert call(pb, **{name: None}) == sa.SA_E_INVALID, name
    assert call(pb, ws=None) == sa.SA_E_WORKSPACE
    need = _bws(2, 100, 128, 512, 0)[1]
    assert call(pb, wsb=need - 1) == sa.SA_E_WORKSPACE
    assert call(_lib.problem(2, 100, 128, 512, 0, 4)) == sa.SA_E_INVALID   # unknown flag bit
    assert call(_lib.problem(2, 100, 128, 512, sa.SA_F32)) == sa.SA_E_UNSUPPORTED
    assert _lib.load().sa_compress_backward_with_sbar(None, *([None] * 14), 0, None, None) == sa.SA_E_INVALID


def test_sbar_binding_validates_before_library():
    import torch
    H = torch.zeros(4, 128, dtype=torch.bfloat16)
    off = torch.tensor([0, 4])
    with pytest.raises(ValueError):   # sbar without mass
        sa.compress_backward(H, off, H[:0], H[:0], H[:0], torch.zeros(1, 1, 128), sbar=torch.zeros(1, 1, 128))


def test_misaligned_inputs_rejected_before_launch():
    """H, Wk, Wv and P are read in 16-byte vectors and offsets as int64: a
    misaligned pointer is an argument error, caught on the host."""
    pb = _lib.problem(2, 100, 128, 512, 0)
    for name in ("H", "Wk", "Wv", "P"):
        assert _call(pb, **{name: FAKE + 2}) == sa.SA_E_INVALID, name
        assert _bcall(pb, **{name: FAKE + 8}) == sa.SA_E_INVALID, name
    assert _call(pb, off=FAKE + 4) == sa.SA_E_INVALID
    assert _bcall(pb, off=FAKE + 4) == sa.SA_E_INVALID


def test_probe_rejects_bad_arguments():
    """sa_probe_mfma checks its arguments on the host before any launch."""
    lib = _lib.load()
    sink = ctypes.c_void_p(16)   # never dereferenced: every call below fails its checks
    assert lib.sa_probe_mfma(2, 10, None, None) == sa.SA_E_INVALID
    assert lib.sa_probe_mfma(3, 10, sink, None) == sa.SA_E_INVALID
    assert lib.sa_probe_mfma(-1, 10, sink, None) == sa.SA_E_INVALID
    assert lib.sa_probe_mfma(2, 0, sink, None) == sa.SA_E_INVALID
    assert lib.sa_probe_mfma(2, 1000001, sink, None) == sa.SA_E_INVALID
