"""The C-ABI library on the host (CPU only; no call here reaches the GPU).

Checks that libsv.so loads, exports every function include/sv.h declares, answers the host-only
queries, and rejects invalid arguments with the documented status before launching anything.
"""
import ctypes
import os
import re

import pytest

import lossless_draft_verification_sv_amd as sv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sv.LIBRARY_PATH):
        pytest.skip("libsv.so not built")
    return sv.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"sv_verify_batch", "sv_verify_greedy", "sv_workspace_bytes"} <= set(names)
    raw = ctypes.CDLL(sv.LIBRARY_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    for code in (sv.SV_OK, sv.SV_ERR_INVALID_ARG, sv.SV_ERR_UNSUPPORTED, sv.SV_ERR_WORKSPACE,
                 sv.SV_ERR_HIP):
        assert sv.sv_status_string(code)
    assert sv.sv_status_string(12345) == "unknown status"


def test_workspace_bytes(lib):
    assert sv.sv_workspace_bytes(0, 8, 100) == 0
    assert sv.sv_workspace_bytes(1, 0, 100) == 0
    assert sv.sv_workspace_bytes(1, 65, 100) == 0
    assert sv.sv_workspace_bytes(1, 8, 0) == 0
    assert sv.sv_workspace_bytes((1 << 20) + 1, 8, 100) == 0
    a = sv.sv_workspace_bytes(64, 8, 151936)
    b = sv.sv_workspace_bytes(256, 16, 151936)
    assert 0 < a < 64 << 20 and 0 < b < 64 << 20
    assert a % 256 == 0


FAKE = 0x1000  # never dereferenced: every call below fails validation first
WS = 0x2000


def call_batch(lib, **kw):
    args = dict(target=FAKE, draft=FAKE, dtype=sv.SV_DTYPE_BF16, B=2, K=4, V=1000,
                temperature=1.0, tokens=FAKE, num_draft=None, uniforms=FAKE, residual=FAKE,
                acc=FAKE, com=FAKE, tp=FAKE, dp=None, ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_batch(*args.values())


def call_greedy(lib, **kw):
    args = dict(target=FAKE, dtype=sv.SV_DTYPE_F32, B=2, K=4, V=1000, tokens=FAKE,
                num_draft=None, acc=FAKE, com=FAKE, ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_greedy(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG),
    (dict(B=(1 << 20) + 1), sv.SV_ERR_INVALID_ARG),
    (dict(K=0), sv.SV_ERR_INVALID_ARG),
    (dict(K=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=0), sv.SV_ERR_INVALID_ARG),
    (dict(dtype=7), sv.SV_ERR_INVALID_ARG),
    (dict(target=None), sv.SV_ERR_INVALID_ARG),
    (dict(draft=None), sv.SV_ERR_INVALID_ARG),
    (dict(tokens=None), sv.SV_ERR_INVALID_ARG),
    (dict(uniforms=None), sv.SV_ERR_INVALID_ARG),
    (dict(residual=None), sv.SV_ERR_INVALID_ARG),
    (dict(acc=None), sv.SV_ERR_INVALID_ARG),
    (dict(com=None), sv.SV_ERR_INVALID_ARG),
    (dict(tp=None), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=0.0), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=-1.0), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=float("nan")), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=float("inf")), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=1e-9), sv.SV_ERR_INVALID_ARG),
    (dict(ws=None), sv.SV_ERR_WORKSPACE),
    (dict(ws=WS + 4), sv.SV_ERR_WORKSPACE),
    (dict(ws=WS + 128), sv.SV_ERR_WORKSPACE),
    (dict(ws_bytes=16), sv.SV_ERR_WORKSPACE),
])
def test_batch_rejects_invalid_arguments(lib, kw, status):
    assert call_batch(lib, **kw) == status
    assert sv.sv_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG),
    (dict(K=0), sv.SV_ERR_INVALID_ARG),
    (dict(K=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=(1 << 26) + 1), sv.SV_ERR_INVALID_ARG),
    (dict(dtype=-1), sv.SV_ERR_INVALID_ARG),
    (dict(target=None), sv.SV_ERR_INVALID_ARG),
    (dict(tokens=None), sv.SV_ERR_INVALID_ARG),
    (dict(acc=None), sv.SV_ERR_INVALID_ARG),
    (dict(com=None), sv.SV_ERR_INVALID_ARG),
    (dict(ws=None), sv.SV_ERR_WORKSPACE),
    (dict(ws_bytes=0), sv.SV_ERR_WORKSPACE),
])
def test_greedy_rejects_invalid_arguments(lib, kw, status):
    assert call_greedy(lib, **kw) == status
    assert sv.sv_last_error() != ""


def call_ragged(lib, **kw):
    args = dict(target=FAKE, draft=FAKE, dtype=sv.SV_DTYPE_BF16, B=2, K=4, V=1000, rows_t=10,
                rows_d=8, t_start=FAKE, d_start=FAKE, num_draft=FAKE, temperature=FAKE,
                tokens=FAKE, uniforms=FAKE, residual=FAKE, acc=FAKE, com=FAKE, tp=FAKE, dp=None,
                ws=WS, ws_bytes=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_ragged(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG),
    (dict(K=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=0), sv.SV_ERR_INVALID_ARG),
    (dict(dtype=3), sv.SV_ERR_INVALID_ARG),
    (dict(target=None), sv.SV_ERR_INVALID_ARG),
    (dict(t_start=None), sv.SV_ERR_INVALID_ARG),
    (dict(d_start=None), sv.SV_ERR_INVALID_ARG),
    (dict(num_draft=None), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=None), sv.SV_ERR_INVALID_ARG),
    (dict(tokens=None), sv.SV_ERR_INVALID_ARG),
    (dict(uniforms=None), sv.SV_ERR_INVALID_ARG),
    (dict(residual=None), sv.SV_ERR_INVALID_ARG),
    (dict(acc=None), sv.SV_ERR_INVALID_ARG),
    (dict(com=None), sv.SV_ERR_INVALID_ARG),
    (dict(tp=None), sv.SV_ERR_INVALID_ARG),
    (dict(rows_t=0), sv.SV_ERR_INVALID_ARG),
    (dict(rows_d=-1), sv.SV_ERR_INVALID_ARG),
    (dict(draft=None), sv.SV_ERR_INVALID_ARG),
    (dict(ws=None), sv.SV_ERR_WORKSPACE),
    (dict(ws=WS + 8), sv.SV_ERR_WORKSPACE),
    (dict(ws_bytes=32), sv.SV_ERR_WORKSPACE),
])
def test_ragged_rejects_invalid_arguments(lib, kw, status):
    assert call_ragged(lib, **kw) == status
    assert sv.sv_last_error() != ""


def test_workspace_size_is_exactly_enough(lib):
    need = sv.sv_workspace_bytes(2, 4, 1000)
    assert call_batch(lib, ws_bytes=need - 1) == sv.SV_ERR_WORKSPACE
    assert call_greedy(lib, ws_bytes=need - 1) == sv.SV_ERR_WORKSPACE


def test_python_binding_rejects_bad_tensors():
    import torch

    t = torch.zeros(2, 5, 10)
    with pytest.raises(ValueError):
        sv.sv_verify_batch(t, torch.zeros(2, 4, 10), torch.zeros(2, 4, dtype=torch.int32),
                           torch.zeros(2, 4), torch.zeros(2))  # CPU tensors
    with pytest.raises((TypeError, ValueError)):
        sv.sv_verify_greedy(torch.zeros(2, 5, 10, dtype=torch.float64),
                            torch.zeros(2, 4, dtype=torch.int32))


def test_read_probe_rejects_invalid_arguments(lib):
    buf = (ctypes.c_uint8 * 64)()
    base = ctypes.addressof(buf)
    aligned = base + (-base) % 16
    out = (ctypes.c_uint32 * 4)()
    probe = ctypes.CDLL(sv.LIBRARY_PATH).sv_read_probe
    probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                      ctypes.c_void_p]
    probe.restype = ctypes.c_int
    assert probe(None, 16, ctypes.addressof(out), 4, None) == sv.SV_ERR_INVALID_ARG
    assert probe(aligned, 16, None, 4, None) == sv.SV_ERR_INVALID_ARG
    assert probe(aligned + 4, 16, ctypes.addressof(out), 4, None) == sv.SV_ERR_INVALID_ARG
    assert probe(aligned, 12, ctypes.addressof(out), 4, None) == sv.SV_ERR_INVALID_ARG
    assert probe(aligned, 16, ctypes.addressof(out), 0, None) == sv.SV_ERR_INVALID_ARG
    assert "16-byte" in sv.sv_last_error() or "groups" in sv.sv_last_error()


@pytest.mark.parametrize("kw", [dict(B=0), dict(K=0), dict(K=65), dict(B=4097, K=1),
                                dict(B=257, K=16), dict(conf=None), dict(num=None),
                                dict(T=16), dict(table=None, threshold=float("nan"))])
def test_schedule_rejects_invalid_arguments(lib, kw):
    args = dict(conf=FAKE, B=4, K=4, table=FAKE, T=4 + 16 + 1, threshold=0.5, num=FAKE,
                ts=None, ds=None, summary=None, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    assert lib.sv_schedule_prefix(*args.values()) == sv.SV_ERR_INVALID_ARG
    assert sv.sv_last_error() != ""


@pytest.mark.parametrize("kw", [dict(ws=None), dict(ws=WS + 4), dict(ws_bytes=8)])
def test_schedule_checks_its_workspace_in_hardware_aware_mode(lib, kw):
    args = dict(conf=FAKE, B=4, K=4, table=FAKE, T=4 + 16 + 1, threshold=0.5, num=FAKE,
                ts=None, ds=None, summary=None, ws=WS, ws_bytes=1 << 20, stream=None)
    args.update(kw)
    assert lib.sv_schedule_prefix(*args.values()) == sv.SV_ERR_WORKSPACE
    assert "workspace" in sv.sv_last_error()


def test_schedule_workspace_size(lib):
    # ceil(B*K / 8) ranking work-groups, three 8-byte words each, rounded up to 256 bytes
    assert lib.sv_schedule_workspace_bytes(256, 16) == 512 * 24
    assert lib.sv_schedule_workspace_bytes(1, 1) == 256
    assert lib.sv_schedule_workspace_bytes(4096, 1) == 512 * 24
    assert lib.sv_schedule_workspace_bytes(3, 5) == 256
    assert lib.sv_schedule_workspace_bytes(0, 4) == 0
    assert lib.sv_schedule_workspace_bytes(4, 65) == 0
    assert lib.sv_schedule_workspace_bytes(4097, 1) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG), (dict(K=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=0), sv.SV_ERR_INVALID_ARG), (dict(dtype=9), sv.SV_ERR_INVALID_ARG),
    (dict(R=8), sv.SV_ERR_INVALID_ARG), (dict(R=264), sv.SV_ERR_INVALID_ARG),
    (dict(R=2048), sv.SV_ERR_INVALID_ARG), (dict(base=None), sv.SV_ERR_INVALID_ARG),
    (dict(left=None), sv.SV_ERR_INVALID_ARG), (dict(tokens=None), sv.SV_ERR_INVALID_ARG),
    (dict(left=FAKE + 8), sv.SV_ERR_INVALID_ARG), (dict(ws=None), sv.SV_ERR_WORKSPACE),
    (dict(ws_bytes=8), sv.SV_ERR_WORKSPACE), (dict(ws=WS + 16), sv.SV_ERR_WORKSPACE),
])
def test_markov_rejects_invalid_arguments(lib, kw, status):
    args = dict(base=FAKE, dtype=sv.SV_DTYPE_BF16, B=4, K=4, V=1000, left=FAKE, right=FAKE,
                R=256, anchor=None, tokens=FAKE, logits=None, ws=WS, ws_bytes=1 << 30,
                stream=None)
    args.update(kw)
    assert lib.sv_markov_draft(*args.values()) == status
    assert sv.sv_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG), (dict(K=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=0), sv.SV_ERR_INVALID_ARG), (dict(dtype=9), sv.SV_ERR_INVALID_ARG),
    (dict(R=264), sv.SV_ERR_INVALID_ARG), (dict(R=272), sv.SV_ERR_INVALID_ARG),
    (dict(kc=0), sv.SV_ERR_INVALID_ARG), (dict(kc=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=10, kc=11), sv.SV_ERR_INVALID_ARG), (dict(V=1 << 26, kc=64), sv.SV_ERR_UNSUPPORTED),
    (dict(base=None), sv.SV_ERR_INVALID_ARG), (dict(tokens=None), sv.SV_ERR_INVALID_ARG),
    (dict(right=FAKE + 4), sv.SV_ERR_INVALID_ARG), (dict(ws=None), sv.SV_ERR_WORKSPACE),
    (dict(ws_bytes=8), sv.SV_ERR_WORKSPACE), (dict(ws=WS + 16), sv.SV_ERR_WORKSPACE),
])
def test_markov_topk_rejects_invalid_arguments(lib, kw, status):
    args = dict(base=FAKE, dtype=sv.SV_DTYPE_BF16, B=4, K=4, V=1000, left=FAKE, right=FAKE,
                R=256, kc=64, anchor=None, tokens=FAKE, cands=None, logits=None, ws=WS,
                ws_bytes=1 << 40, stream=None)
    args.update(kw)
    assert lib.sv_markov_topk(*args.values()) == status
    assert sv.sv_last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), sv.SV_ERR_INVALID_ARG), (dict(K=65), sv.SV_ERR_INVALID_ARG),
    (dict(V=0), sv.SV_ERR_INVALID_ARG), (dict(dtype=9), sv.SV_ERR_INVALID_ARG),
    (dict(R=8), sv.SV_ERR_INVALID_ARG), (dict(R=2048), sv.SV_ERR_INVALID_ARG),
    (dict(base=None), sv.SV_ERR_INVALID_ARG), (dict(tau=None), sv.SV_ERR_INVALID_ARG),
    (dict(uni=None), sv.SV_ERR_INVALID_ARG), (dict(tokens=None), sv.SV_ERR_INVALID_ARG),
    (dict(logits=None), sv.SV_ERR_INVALID_ARG), (dict(right=FAKE + 8), sv.SV_ERR_INVALID_ARG),
    (dict(ws=None), sv.SV_ERR_WORKSPACE), (dict(ws_bytes=8), sv.SV_ERR_WORKSPACE),
    (dict(ws=WS + 16), sv.SV_ERR_WORKSPACE), (dict(R=1040), sv.SV_ERR_INVALID_ARG),
])
def test_markov_sampled_rejects_invalid_arguments(lib, kw, status):
    args = dict(base=FAKE, dtype=sv.SV_DTYPE_BF16, B=4, K=4, V=1000, left=FAKE, right=FAKE,
                R=256, anchor=None, tau=FAKE, uni=FAKE, tokens=FAKE, logits=FAKE, ws=WS,
                ws_bytes=1 << 30, stream=None)
    args.update(kw)
    assert lib.sv_markov_draft_sampled(*args.values()) == status
    assert sv.sv_last_error() != ""


def test_markov_workspace_holds_the_draw_decisions():
    lib = sv.load_library()
    for B, V in [(1, 5), (64, 151936), (64, 100), (200, 151936), (100, 1000)]:
        ntile = -(-V // 64)
        Bl = min(B, 64)
        one_launch = Bl * (ntile + Bl) * 16 + Bl * 8 + Bl * 16
        assert lib.sv_markov_workspace_bytes(B, V) >= max(one_launch, B * ntile * 8)


def test_noalloc_validates_before_any_gpu_call(lib):
    """The allocation-free entry point rejects a batch whose scratch would exceed the 16 MiB it
    holds per GPU, and invalid shapes, before it looks anything up on a device."""
    need = sv.sv_workspace_bytes(4096, 64, 151936)
    assert need > 16 << 20
    st = lib.sv_verify_batch_noalloc(FAKE, FAKE, sv.SV_DTYPE_BF16, 4096, 64, 151936, 1.0, FAKE,
                                     None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == sv.SV_ERR_UNSUPPORTED and "16777216" in sv.sv_last_error()
    st = lib.sv_verify_batch_noalloc(FAKE, FAKE, sv.SV_DTYPE_BF16, 0, 8, 1000, 1.0, FAKE, None,
                                     FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert st == sv.SV_ERR_INVALID_ARG
