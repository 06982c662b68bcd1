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
    assert names == {"gmla_probe_mfma", "gmla_probe_mfma_random", "gmla_probe_read"}
    lib = ctypes.CDLL(os.path.join(ROOT, "causal_softmax_attention_gmla_amd", "libgmla_probe.so"))
    for n in names:
        assert hasattr(lib, n)
    lib.gmla_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.gmla_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gmla_probe_read(FAKE, 1000, 8, FAKE, None) == -1  # not a multiple of the chunk
    assert lib.gmla_probe_mfma(0, 10, FAKE, None) == -1
    lib.gmla_probe_mfma_random.argtypes = lib.gmla_probe_mfma.argtypes
    assert lib.gmla_probe_mfma_random(4, 0, FAKE, None) == -1


def test_status_strings_and_version():
    lib = gm.library()
    assert lib.gmla_version() >= 100
    for code, name in ((0, b"GMLA_OK"), (-1, b"GMLA_ERR_INVALID_ARG"), (-2, b"GMLA_ERR_UNSUPPORTED"),
                       (-3, b"GMLA_ERR_WORKSPACE"), (-4, b"GMLA_ERR_HIP"), (-5, b"GMLA_ERR_TOO_LARGE"),
                       (99, b"GMLA_ERR_UNKNOWN")):
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


MAX_KEYS = 2 ** 31 - 1 - 2 ** 14  # longest sequence the 32-bit row indices take


def test_prefill_rejects_key_stride_past_2_24():
    """The MFMA kernel's byte offsets inside one 64-row key tile are 32-bit: a token
    stride of 2^24 elements or more is unsupported (2^24 - 8 is the largest accepted)."""
    big = (ctypes.c_int64 * 3)(2 ** 30, 2 ** 24, 128)
    assert _prefill(strides=big) == -2
    assert _chunk(kv_strides=big) == -2


def test_sequence_lengths_past_the_32_bit_row_limit_are_unsupported():
    assert _prefill(T=MAX_KEYS + 1) == -2
    assert _chunk(Tq=8, Tk=MAX_KEYS + 1) == -2
    assert _decode(N=MAX_KEYS + 1) == -2
    assert _decode(N=2 ** 31 - 1) == -2


def test_decode_noalloc_limits():
    """The no-allocation decode keeps its split partials in a fixed 4 MiB array: partials
    beyond it are rejected before any HIP call; validation matches the workspace decode."""
    lib = gm.library()
    cap = lib.gmla_decode_noalloc_scratch_bytes()
    assert cap == 4 << 20
    B, H, N = 8, 96, 4096
    assert lib.gmla_decode_workspace_bytes(B, H, N, 128, 4096) > cap
    assert _noalloc(B=B, H=H, N=N, splits=4096) == -5
    assert _noalloc(N=0) == -1
    assert _noalloc(D=48) == -2
    assert _noalloc(N=MAX_KEYS + 1) == -2
    assert _noalloc(K=ctypes.c_void_p((1 << 20) + 2)) == -1
    # every automatic split choice fits: at most (2048 + B*H - 1) slots of D + 2 floats
    for B, H, N in ((4, 96, 131072), (1, 1, 10 ** 9), (1, 96, 2 ** 30), (2, 1023, 10 ** 8)):
        s = lib.gmla_decode_num_splits(B, H, N, 128)
        assert lib.gmla_decode_workspace_bytes(B, H, N, 128, s) <= cap


def _varlen(**kw):
    a = dict(dtype=1, B=2, H=4, D=128, scale=0.1, causal=1, Q=FAKE, q_strides=None, cu_q=FAKE,
             max_q=100, K=FAKE, V=FAKE, kv_strides=None, cu_k=FAKE, max_k=300, G=None, O=FAKE,
             stream=None)
    a.update(kw)
    return gm.library().gmla_attend_varlen(*a.values())


@pytest.mark.parametrize("bad", [dict(B=0), dict(H=0), dict(max_q=0), dict(max_k=-1), dict(causal=3),
                                 dict(cu_q=None), dict(cu_k=None), dict(cu_q=ctypes.c_void_p((1 << 20) + 2)),
                                 dict(Q=None), dict(O=None), dict(scale=float("nan")),
                                 dict(q_strides=(ctypes.c_int64 * 2)(512 + 4, 128)),
                                 dict(kv_strides=(ctypes.c_int64 * 2)(-512, 128))])
def test_varlen_rejects_bad_arguments(bad):
    assert _varlen(**bad) == -1


def test_varlen_limits():
    assert _varlen(D=96) == -2
    assert _varlen(max_q=MAX_KEYS + 1) == -2
    assert _varlen(max_k=MAX_KEYS + 1) == -2
    assert _varlen(kv_strides=(ctypes.c_int64 * 2)(2 ** 24, 128)) == -2


def _decode_varlen(**kw):
    a = dict(dtype=1, B=2, H=4, N=100, D=128, scale=0.1, Q=FAKE, K=FAKE, V=FAKE, kv_strides=None,
             lens=FAKE, G=None, O=FAKE, ws=None, ws_bytes=0, splits=1, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_decode_varlen(*a.values())


def test_decode_varlen_arguments():
    assert _decode_varlen(lens=None) == -1
    assert _decode_varlen(lens=ctypes.c_void_p((1 << 20) + 1)) == -1
    assert _decode_varlen(N=0) == -1
    assert _decode_varlen(D=48) == -2
    assert _decode_varlen(splits=4) == -3


def _platent(**kw):
    a = dict(dtype=1, B=1, T=300, H=2, D=128, d_c=512, scale=0.1, causal=1, Q=FAKE, q_strides=None,
             C=FAKE, W_k=FAKE, W_v=FAKE, G=None, O=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_prefill_latent(*a.values())


def test_prefill_latent_arguments():
    lib = gm.library()
    need = lib.gmla_prefill_latent_workspace_bytes(1, 300, 2, 128)
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert need == 2 * r256(300 * 2 * 128 * 2) + 4 * (2 * 3 + 8 + 1)
    for bad in (dict(B=0), dict(T=0), dict(causal=2), dict(Q=None), dict(C=None), dict(O=None),
                dict(scale=0.0), dict(C=ctypes.c_void_p((1 << 20) + 8)),
                dict(q_strides=(ctypes.c_int64 * 3)(300 * 256, 256 + 4, 128))):
        assert _platent(**bad) == -1, bad
    assert _platent(dtype=0) == -2
    assert _platent(d_c=100) == -2
    assert _platent(D=64) == -2
    assert _platent(T=MAX_KEYS + 1) == -2
    assert _platent(ws=None) == -3
    assert _platent(ws_bytes=need - 1) == -3
    assert _platent(ws=ctypes.c_void_p((1 << 20) + 16)) == -3


def _latent(**kw):
    a = dict(dtype=1, B=2, H=4, N=100, D=128, d_c=512, scale=0.1, Q=FAKE, C=FAKE, c_strides=None,
             W_k=FAKE, W_v=FAKE, G=None, O=FAKE, ws=FAKE, ws_bytes=1 << 30, splits=0, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_decode_latent(*a.values())


@pytest.mark.parametrize("bad", [dict(B=0), dict(N=0), dict(H=0), dict(Q=None), dict(C=None),
                                 dict(W_v=None), dict(O=None), dict(scale=0.0), dict(splits=-1),
                                 dict(C=ctypes.c_void_p((1 << 20) + 8)),
                                 dict(c_strides=(ctypes.c_int64 * 2)(100 * 512, 516)),
                                 dict(c_strides=(ctypes.c_int64 * 2)(-512, 512))])
def test_decode_latent_rejects_bad_arguments(bad):
    assert _latent(**bad) == -1


def test_decode_latent_limits_and_workspace():
    lib = gm.library()
    assert _latent(dtype=0) == -2                    # bf16 only
    assert _latent(D=64) == -2
    assert _latent(d_c=64) == -2 and _latent(d_c=384) == -2
    assert _latent(N=MAX_KEYS + 1) == -2
    assert _latent(c_strides=(ctypes.c_int64 * 2)(2 ** 40, 2 ** 25)) == -2
    need = lib.gmla_decode_latent_workspace_bytes(2, 4, 100, 512, 0)
    assert need > 0
    assert _latent(ws=None) == -3
    assert _latent(ws_bytes=need - 1) == -3
    assert _latent(ws=ctypes.c_void_p((1 << 20) + 16)) == -3  # not 256-byte aligned
    # ranges are rounded to 32-row tiles: the count used covers N with none empty
    for B, H, N in ((8, 96, 1001), (4, 96, 131072), (1, 1, 1), (1, 40, 33), (2, 3, 100000)):
        s = lib.gmla_decode_latent_num_splits(B, H, N, 512)
        kps = -(-N // s)
        assert s >= 1 and (s - 1) * (-(-kps // 32) * 32) < N
    assert lib.gmla_decode_latent_num_splits(8, 96, 1001, 512) == 7
    # workspace: absorbed queries (bf16), (m, l) and d_c sums per (b, h, range)
    s = lib.gmla_decode_latent_num_splits(8, 96, 1001, 512)
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert lib.gmla_decode_latent_workspace_bytes(8, 96, 1001, 512, 0) == \
        r256(768 * 512 * 2) + r256(768 * s * 8) + 768 * s * 512 * 4


def _latent_varlen(**kw):
    a = dict(dtype=1, B=2, H=4, N=100, D=128, d_c=512, scale=0.1, Q=FAKE, C=FAKE, c_strides=None,
             lens=FAKE, W_k=FAKE, W_v=FAKE, G=None, O=FAKE, ws=FAKE, ws_bytes=1 << 30, splits=0,
             stream=None)
    a.update(kw)
    return gm.library().gmla_attend_decode_latent_varlen(*a.values())


def test_decode_latent_varlen_arguments():
    assert _latent_varlen(lens=None) == -1
    assert _latent_varlen(lens=ctypes.c_void_p((1 << 20) + 2)) == -1  # not 4-byte aligned
    assert _latent_varlen(N=0) == -1
    assert _latent_varlen(C=None) == -1
    assert _latent_varlen(d_c=384) == -2
    assert _latent_varlen(N=MAX_KEYS + 1) == -2
    assert _latent_varlen(ws=None) == -3


def _noalloc(**kw):
    a = dict(dtype=1, B=2, H=4, N=100, D=128, scale=0.1, Q=FAKE, K=FAKE, V=FAKE, kv_strides=None,
             G=None, O=FAKE, splits=1, stream=None)
    a.update(kw)
    return gm.library().gmla_attend_decode_noalloc(*a.values())


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


def test_gate_out_workspace_size_and_overlap():
    lib = gm.library()
    # bf16 with d_model a multiple of 64 takes the gate pass + LDS GEMM; others need nothing
    assert lib.gmla_gate_out_workspace_bytes(1, 2048, 12288) == 2048 * 12288 * 2
    assert lib.gmla_gate_out_workspace_bytes(1, 3, 64) == 3 * 64 * 2
    assert lib.gmla_gate_out_workspace_bytes(0, 2048, 12288) == 0
    assert lib.gmla_gate_out_workspace_bytes(1, 2048, 100) == 0
    assert lib.gmla_gate_out_workspace_bytes(1, 0, 128) == 0
    # a workspace overlapping an operand is rejected before anything launches
    M, dm = 64, 128
    mat = M * dm * 2
    G, O, W, Y = (ctypes.c_void_p((1 << 24) * (i + 1)) for i in range(4))
    for start in (G.value - 16, O.value + mat - 16, W.value, Y.value + 4096):
        ws = ctypes.c_void_p(start)
        assert lib.gmla_gate_out_ws(1, M, dm, G, O, W, Y, ws, mat, None) == -1, hex(start)
    # invalid arguments are still caught with a workspace
    assert lib.gmla_gate_out_ws(1, 4, 16, None, None, None, FAKE, FAKE, 1 << 20, None) == -1


def test_linear_split_k_plan_and_arguments():
    lib = gm.library()
    # the latent down-projection splits its 12288-deep reduction; wide or shallow products do not
    assert lib.gmla_linear_workspace_bytes(2048, 512, 12288) == 8 * 2048 * 512 * 4
    assert lib.gmla_linear_workspace_bytes(2048, 12288, 12288) == 0
    assert lib.gmla_linear_workspace_bytes(2048, 24576, 512) == 0
    assert lib.gmla_linear_workspace_bytes(2048, 512, 512) == 0
    assert lib.gmla_linear_ws(1, 4, 4, 12, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.gmla_linear_ws(1, 0, 4, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert lib.gmla_linear_ws(3, 4, 4, 8, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1


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


NO_DEVICE_SCRIPT = r"""
import ctypes, sys
try:
    hip = ctypes.CDLL("libamdhip64.so")
except OSError:
    hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
n = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(n)) == 0 and n.value > 0:
    sys.exit(77)  # a device is visible: the fake pointers below must never reach it
sys.path.insert(0, sys.argv[1])
import test_boundary as tb
tb.valid_calls_without_a_device()
print("no-device calls ok")
"""


def valid_calls_without_a_device():
    """Arguments that pass validation reach the launch; with no HIP device the launch
    fails and the call returns GMLA_ERR_HIP instead of crashing."""
    lib = gm.library()
    assert _prefill() == -4
    assert _chunk() == -4
    assert _decode() == -4
    assert _noalloc() == -4
    assert _noalloc(splits=4) == -4  # the scratch lookup fails without a device
    assert _latent() == -4
    assert _latent_varlen() == -4
    assert _platent() == -4
    assert lib.gmla_linear_ws(1, 2048, 512, 12288, FAKE, FAKE, FAKE, FAKE, 1 << 26, None) == -4
    assert lib.gmla_linear_ws(1, 64, 64, 64, FAKE, FAKE, FAKE, None, 0, None) == -4
    assert _varlen() == -4
    assert _varlen(dtype=0, D=64) == -4
    assert _decode_varlen() == -4
    assert lib.gmla_linear(1, 64, 64, 64, FAKE, FAKE, FAKE, None) == -4
    assert lib.gmla_latent_expand(1, 64, 64, 128, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -4
    assert lib.gmla_gate_out(1, 64, 128, FAKE, FAKE, FAKE, FAKE, None) == -4
    ws = ctypes.c_void_p(1 << 30)
    assert lib.gmla_gate_out_ws(1, 64, 128, FAKE, FAKE, FAKE, FAKE, ws, 64 * 128 * 2, None) == -4


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path only")
def test_valid_call_without_a_device_returns_hip_error():
    """Runs the fake-pointer calls in a child process whose environment hides every
    device, and which exits before them if a device is visible anyway."""
    import subprocess
    import sys

    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", NO_DEVICE_SCRIPT, os.path.join(ROOT, "tests")],
                       capture_output=True, text=True, env=env, timeout=300,
                       cwd=ROOT)
    if r.returncode == 77:
        pytest.skip("a HIP device is visible")
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "no-device calls ok" in r.stdout


def _bench_module():
    import importlib.util
    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(here, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_bench_range_labels_match_the_library_plan():
    """The latent range sweep labels each run with the range count the library uses for a
    requested count; that count is read back here from the workspace size the library
    asks for (absorbed queries, then (m, l) and d_c sums per range)."""
    bench = _bench_module()
    lib = gm.library()
    B, H, dc = 8, 96, 512
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for N in (1, 31, 33, 1001, 4100, 131072):
        for req in (1, 2, 3, 4, 7, 8, 10, 16, 1000):
            ws = lib.gmla_decode_latent_workspace_bytes(B, H, N, dc, req)
            used = bench.lib_ranges(N, req)
            assert ws == r256(B * H * dc * 2) + r256(B * H * used * 8) + B * H * used * dc * 4, (N, req)


def test_bench_source_digest_ignores_comments_only(tmp_path):
    """Recorded counters stay valid across comment edits and are voided by code edits."""
    bench = _bench_module()
    src = tmp_path / "k.hip"
    bench.HERE = str(tmp_path)
    bench.KERNEL_SOURCES = {"k": ["k.hip"]}
    src.write_text("int a = 1;  // one\n\n// note\nint b = 2;\n")
    d0 = bench.source_digest("k")
    src.write_text("int a = 1;  // changed comment\n// another note\n\nint b = 2;\n")
    assert bench.source_digest("k") == d0
    src.write_text("int a = 1;\nint b = 3;\n")
    assert bench.source_digest("k") != d0
