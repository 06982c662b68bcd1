"""The decode entry point that allocates nothing (gmla_attend_decode_noalloc), called
through the C ABI, against gmla_attend_decode with a caller workspace: two calls in a
row on the fixed scratch array, the second smaller than the first, each equal to the
workspace call's output (same kernels, same splits: bitwise) and so within the
per-row bf16 bar against it."""
import ctypes

import numpy as np
import pytest
import torch

import causal_softmax_attention_gmla_amd as gm
from causal_softmax_attention_gmla_amd import inputs as I
from gpu_helpers import announce, check_f32_abs, check_rows_rel, host, need_gpu

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, g, out, splits):
    B, H, N, D = k.shape
    lib = gm.library()
    dt = gm.GMLA_BF16 if q.dtype == torch.bfloat16 else gm.GMLA_F32
    strides = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gmla_attend_decode_noalloc(dt, B, H, N, D, float(D ** -0.5), p(q), p(k), p(v),
                                          strides, p(g), p(out), splits, stream)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_noalloc_matches_workspace_decode(dtype):
    dev = need_gpu()
    lib = gm.library()
    # first call: 384 heads of 20000 keys in 6 splits (auto), partials in the scratch array;
    # second call smaller (16 heads, 3000 keys, 3 splits, gated): it reuses the array,
    # whose tail still holds the first call's partials
    for B, H, N, splits, gate in ((4, 96, 20000, 0, False), (2, 8, 3000, 3, True)):
        announce(f"decode noalloc {dtype} B={B} H={H} N={N} splits={splits}")
        q, k, v, g = I.decode_inputs(B, H, N, 128, dtype, dev, seed=8800 + N, gate=gate)
        used = splits or lib.gmla_decode_num_splits(B, H, N, 128)
        assert used > 1
        assert lib.gmla_decode_workspace_bytes(B, H, N, 128, used) <= \
            lib.gmla_decode_noalloc_scratch_bytes()
        ref = gm.attend_decode(q, k, v, g, num_splits=splits)
        out = torch.full((B, H * 128), float("nan"), dtype=dtype, device=dev)
        assert _noalloc(q, k, v, g, out, splits) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        if dtype == torch.float32:
            check_f32_abs(host(out), host(ref))
        else:
            check_rows_rel(host(out), host(ref), 128)


def test_decode_noalloc_rejects_oversized_partials():
    """Partials larger than the fixed array: GMLA_ERR_TOO_LARGE, nothing launched."""
    dev = need_gpu()
    lib = gm.library()
    B, H, N = 8, 96, 4096
    need = lib.gmla_decode_workspace_bytes(B, H, N, 128, 4096)
    assert need > lib.gmla_decode_noalloc_scratch_bytes()
    q, k, v, _ = I.decode_inputs(B, H, N, 128, torch.bfloat16, dev, seed=8900)
    out = torch.zeros((B, H * 128), dtype=torch.bfloat16, device=dev)
    assert _noalloc(q, k, v, None, out, 4096) == -5
    torch.cuda.synchronize()
    assert not out.any()
    assert np.all(host(out) == 0)
