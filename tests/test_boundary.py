"""The C-ABI library on the host (no GPU): it loads, exports every symbol that
include/gmla.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

import causal_softmax_attention_gmla_amd as gm
from causal_softmax_attention_gmla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gmla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gmla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("gmla_attend_prefill", "gmla_attend_decode", "gmla_latent_expand", "gmla_gate_out"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = gm.library()
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in gmla.h but not exported"
    assert set(declared_functions()) == set(_lib.SIGNATURES), "binding signatures out of sync"


def test_probe_library_exports_its_header():
    """The benchmark's measurement aids live in their own library and header."""
    text = open(os.path.join(ROOT, "include", "gmla_probe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(gmla_probe_[a-z0-9_]+)\s*\(", text))
    assert names == {"gmla_probe_mfma", "gmla_probe_read"}
    lib = ctypes.CDLL(os.path.join(ROOT, "causal_softmax_attention_gmla_amd", "libgmla_probe.so"))
    for n in names:
        assert hasattr(lib, n)
    lib.gmla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.gmla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gmla_probe_read(FAKE, 1000, 8, FAKE, None) == -1  # not a multiple of the chunk
    assert lib.gmla_probe_mfma(0, 10, FAKE, None) == -1


def test_status_strings_and_version():
    lib = gm.library()
    assert lib.gmla_version() >= 100
    for code, name in ((0, b"GMLA_OK"), (-1, b"GMLA_ERR_INVALID_ARG"), (-2, b"GMLA_ERR_UNSUPPORTED"),
                       (-3, b"GMLA_ERR_WORKSPACE"), (-4, b"GMLA_ERR_HIP"), (99, b"GMLA_ERR_UNKNOWN")):
        assert lib.gmla_status_string(code) == name


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def _prefill(**kw):
    a = dict(dtype=1, B=1, T=8, H=2, D=128, scale=0.1, causal=1, Q=FAKE, K=FAKE, V=FAKE,
             strides=None, G=None, O=FAKE, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_prefill(*a.values())


@pytest.mark.parametrize("bad", [dict(dtype=7), dict(B=0), dict(T=0), dict(H=-1), dict(D=0),
                                 dict(causal=2), dict(Q=None), dict(O=None), dict(scale=0.0),
                                 dict(scale=float("nan")), dict(Q=ctypes.c_void_p((1 << 20) + 1)),
                                 dict(O=ctypes.c_void_p((1 << 20) + 8))])
def test_prefill_rejects_bad_arguments(bad):
    assert _prefill(**bad) == -1


def test_prefill_unsupported_head_width():
    assert _prefill(D=96) == -2
    assert _prefill(D=256, dtype=0) == -2


def test_prefill_rejects_misaligned_strides():
    s = (ctypes.c_int64 * 3)(8 * 2 * 128, 2 * 128 + 4, 128)
    assert _prefill(strides=s) == -1
    neg = (ctypes.c_int64 * 3)(-1, 256, 128)
    assert _prefill(strides=neg) == -1


def _chunk(**kw):
    a = dict(dtype=1, B=1, Tq=8, Tk=40, H=2, D=128, scale=0.1, causal=1, Q=FAKE, q_strides=None,
             K=FAKE, V=FAKE, kv_strides=None, G=None, O=FAKE, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_chunk(*a.values())


@pytest.mark.parametrize("bad", [dict(Tq=0), dict(Tq=41), dict(Tk=0), dict(B=0), dict(causal=2),
                                 dict(Q=None), dict(K=None), dict(scale=0.0),
                                 dict(q_strides=(ctypes.c_int64 * 3)(-8, 256, 128)),
                                 dict(kv_strides=(ctypes.c_int64 * 3)(40 * 256, 256 + 4, 128))])
def test_chunk_rejects_bad_arguments(bad):
    """A chunk needs 1 <= Tq <= Tk, valid strides (multiples of 8 for the MFMA path)."""
    assert _chunk(**bad) == -1


def test_chunk_wrapper_checks_shapes():
    q = torch.zeros((1, 9, 2, 128), dtype=torch.bfloat16)
    k = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gm.attend_chunk(q, k, k)  # chunk longer than the key sequence
    with pytest.raises(ValueError):
        gm.attend_chunk(q[:, :4], k[:, :, :1], k[:, :, :1])  # head count differs


def _decode(**kw):
    a = dict(dtype=1, B=2, H=4, N=100, D=128, scale=0.1, Q=FAKE, K=FAKE, V=FAKE, kv_strides=None,
             G=None, O=FAKE, ws=None, ws_bytes=0, splits=1, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_decode(*a.values())


@pytest.mark.parametrize("bad", [dict(dtype=-1), dict(N=0), dict(B=0), dict(K=None),
                                 dict(splits=-1), dict(scale=-1.0), dict(K=ctypes.c_void_p((1 << 20) + 2))])
def test_decode_rejects_bad_arguments(bad):
    assert _decode(**bad) == -1


def test_decode_workspace_checks():
    lib = gm.library()
    need = lib.gmla_decode_workspace_bytes(2, 4, 100, 128, 4)
    assert need == 2 * 4 * 4 * 130 * 4
    assert lib.gmla_decode_workspace_bytes(2, 4, 100, 128, 1) == 0
    assert _decode(splits=4) == -3
    assert _decode(splits=4, ws=FAKE, ws_bytes=need - 1) == -3
    assert _decode(D=48) == -2


def test_decode_split_heuristic():
    lib = gm.library()
    for B, H, N in ((8, 96, 1001), (4, 96, 131072), (1, 1, 1), (1, 1, 100000), (64, 96, 50)):
        s = lib.gmla_decode_num_splits(B, H, N, 128)
        assert 1 <= s <= 256 and s <= max(1, N // 1024)
    # the two decode workloads: one split for 1001 keys, six for 131072 keys
    assert lib.gmla_decode_num_splits(8, 96, 1001, 128) == 1
    assert lib.gmla_decode_num_splits(4, 96, 131072, 128) == 6


def test_projection_argument_checks():
    lib = gm.library()
    assert lib.gmla_linear(1, 4, 4, 12, FAKE, FAKE, FAKE, None) == -1  # K % 8 for bf16
    assert lib.gmla_linear(1, 0, 4, 8, FAKE, FAKE, FAKE, None) == -1
    assert lib.gmla_latent_expand(1, 4, 8, 16, FAKE, None, FAKE, FAKE, FAKE, None) == -1
    assert lib.gmla_gate_out(1, 4, 16, None, None, None, FAKE, None) == -1
    assert lib.gmla_gate_out(3, 4, 16, None, FAKE, None, FAKE, None) == -1


def test_binding_rejects_cpu_tensors_and_mismatches():
    import torch
    q = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gm.attend_prefill(q, q, q)
    with pytest.raises(ValueError):
        gm.attend_prefill(q, q[:, :2], q)
    with pytest.raises(TypeError):
        gm.attend_prefill(q, q, q, causal=1)
    x = torch.zeros(1, 4, 6)
    with pytest.raises(ValueError):
        gm.gated_mla(x, *([torch.zeros(6, 6)] * 6), num_heads=4)
    with pytest.raises(TypeError):
        gm.gated_mla(x, *([torch.zeros(6, 6)] * 6), num_heads=2, causal="yes")
    # decode over the latent cache: shape checks come before any device work
    qd = torch.zeros(2, 4, 128, dtype=torch.bfloat16)
    c = torch.zeros(2, 10, 64, dtype=torch.bfloat16)
    w = torch.zeros(4 * 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gm.attend_decode_latent(qd[0], c, w, w)            # q not [B, H, D]
    with pytest.raises(ValueError):
        gm.attend_decode_latent(qd, c[:1], w, w)           # batch sizes differ
    with pytest.raises(ValueError):
        gm.attend_decode_latent(qd, c, w[:256], w[:256])   # up-projections not H*D rows
    with pytest.raises(ValueError):
        gm.attend_decode_latent(qd, c, w, w)               # host tensors


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path only")
def test_valid_call_without_a_device_returns_hip_error():
    """Arguments that pass validation reach the launch; with no HIP device the launch
    fails and the call returns GMLA_ERR_HIP instead of crashing."""
    lib = gm.library()
    assert _prefill() == -4
    assert _chunk() == -4
    assert _decode() == -4
    assert lib.gmla_linear(1, 64, 64, 64, FAKE, FAKE, FAKE, None) == -4
    assert lib.gmla_latent_expand(1, 64, 64, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -4
    assert lib.gmla_gate_out(1, 64, 128, FAKE, FAKE, FAKE, FAKE, None) == -4
